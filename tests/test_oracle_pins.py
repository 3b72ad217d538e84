"""Pins of the fp64 oracle against what the pages and the mathematics fix.

Each test checks the oracle against something other than itself: numbers the pages
print (tests/golden/page_constants.json), closed forms evaluated independently
(Python's decimal module), library routines (torch's casts, rms_norm and
scaled_dot_product_attention), invariants, and a pure-Python loop implementation
of the whole layer on tiny inputs.
"""

import json
import math
import os
import struct
from decimal import Decimal, getcontext
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle.beam_oracle as O
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "page_constants.json")


def golden():
    with open(GOLDEN) as f:
        return json.load(f)


def bits_bf16(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


# ------------------------------------------------------------------ formats

def test_bf16_round_matches_torch_cast():
    rng = np.random.default_rng(11)
    mags = np.exp2(rng.uniform(-140, 127, 200_000))
    x = (mags * rng.choice([-1.0, 1.0], mags.shape)).astype(np.float32)
    # ties: values exactly halfway between two bf16 numbers
    base = rng.integers(0, 1 << 15, 5000).astype(np.uint32) << 16
    ties = (base | np.uint32(0x8000)).view(np.float32)
    x = np.concatenate([x, ties[np.isfinite(ties)], np.float32([0.0, -0.0, 3.3895e38])])
    ours = O.f64_to_bf16_bits(x.astype(np.float64))
    ref = bits_bf16(torch.from_numpy(x).to(torch.bfloat16))
    assert np.array_equal(ours, ref)


def test_bf16_decode_is_exact():
    allbits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    ours = O.bf16_bits_to_f64(allbits)
    ref = torch.from_numpy(allbits.view(np.int16)).view(torch.bfloat16).double().numpy()
    fin = np.isfinite(ref)
    assert np.array_equal(ours[fin], ref[fin])
    assert np.array_equal(np.isnan(ours), np.isnan(ref))


def test_e4m3_decode_all_codes_match_torch():
    codes = np.arange(256, dtype=np.uint8)
    ours = O.e4m3_to_f64(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).double().numpy()
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    fin = ~np.isnan(ref)
    assert np.array_equal(ours[fin], ref[fin])
    assert O.E4M3_MAX == 448.0
    assert np.sum(np.isnan(ours)) == 2  # 0x7F and 0xFF only


def test_e4m3_encode_all_bf16_inputs_match_torch_after_clamp():
    allbits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    vals = O.bf16_bits_to_f64(allbits)
    fin = np.isfinite(vals)
    x = vals[fin]
    ours = O.f64_to_e4m3(x)
    # torch's cast does not saturate (it maps out-of-range values to NaN), so the
    # library reference gets an explicit clamp first.
    ref = torch.from_numpy(np.clip(x, -448, 448)).float().to(torch.float8_e4m3fn)
    ref = ref.view(torch.uint8).numpy()
    # -0 and +0 differ only in the sign bit; both libraries keep the sign.
    assert np.array_equal(ours, ref)


def test_e4m3_saturates_and_roundtrips():
    assert O.f64_to_e4m3([480.0, 1e9, -1e9, 449.0, 464.0, 463.99])[0] == 0x7E
    assert list(O.f64_to_e4m3([480.0, 1e9, -1e9])) == [0x7E, 0x7E, 0xFE]
    assert O.f64_to_e4m3([np.nan])[0] == 0x7F
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    assert np.array_equal(O.f64_to_e4m3(O.e4m3_to_f64(codes)), codes)
    # smallest subnormal 2^-9 and the tie half of it rounds to even (zero)
    assert O.e4m3_to_f64([1])[0] == 2.0 ** -9
    assert O.f64_to_e4m3([2.0 ** -10])[0] == 0
    assert O.f64_to_e4m3([3 * 2.0 ** -10])[0] == 2


# ------------------------------------------------------------------ norm

def test_rms_norm_matches_torch():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((64, 48, 128)) * rng.uniform(0.01, 30, (64, 48, 1))
    w = 1 + 0.1 * rng.standard_normal(128)
    ours = O.rms_norm(x, w, 1e-6)
    ref = torch.nn.functional.rms_norm(torch.from_numpy(x), (128,), torch.from_numpy(w), 1e-6)
    np.testing.assert_allclose(ours, ref.numpy(), rtol=1e-13, atol=1e-13)


def test_rms_norm_closed_form_unit_weight():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((10, 128)) * 1e-3
    y = O.rms_norm(x, np.ones(128), 1e-6)
    ms = np.mean(x * x, axis=-1)
    np.testing.assert_allclose(np.mean(y * y, axis=-1), ms / (ms + 1e-6), rtol=1e-12)
    # scale invariance when mean(x^2) >> eps
    np.testing.assert_allclose(O.rms_norm(x * 1e4, 1.0), O.rms_norm(x * 1e5, 1.0), rtol=1e-7)


# ------------------------------------------------------------------ SSMax

def _dec_pow(base: Decimal, e: Decimal) -> Decimal:
    return (base.ln() * e).exp()


def test_ssmax_closed_forms():
    getcontext().prec = 40
    g = golden()["ssmax"]
    assert (g["base"], g["exponent"], g["position_origin"]) == (2048, 0.1, 1)
    tenth = Decimal(1) / Decimal(10)
    cases = {
        1: _dec_pow(Decimal(2049) / Decimal(2048), tenth),
        2048: _dec_pow(Decimal(2), tenth),                 # 2^0.1
        100000: _dec_pow(Decimal(1) + Decimal(100000) / Decimal(2048), tenth),
        1048576: _dec_pow(Decimal(513), tenth),            # 513^0.1
    }
    for p, ref in cases.items():
        assert abs(float(O.ssmax_scale(p)) - float(ref)) <= 2e-16 * float(ref), p
    # the zero-based form of the SGLang page: position p0 scaled by (1+(p0+1)/2048)^0.1
    p0 = np.arange(0, 5000)
    np.testing.assert_array_equal(O.ssmax_scale(p0 + 1), np.power(1 + (p0 + 1) / 2048.0, 0.1))


def test_prepare_q_full_layer_scales_by_ssmax_of_one_based_position():
    getcontext().prec = 40
    rng = np.random.default_rng(3)
    x = bits_bf16(torch.from_numpy(rng.standard_normal((4, 48, 128)).astype(np.float32)).bfloat16())
    wt = (1 + 0.1 * torch.from_numpy(rng.standard_normal(128).astype(np.float32))).bfloat16()
    w = bits_bf16(wt)
    pos = np.array([0, 1, 2047, 1048575])   # 0-based; p = pos + 1
    q = O.prepare_qk(x, w, pos, "full", True)
    xt = torch.from_numpy(O.bf16_bits_to_f64(x))
    n = torch.nn.functional.rms_norm(xt, (128,), wt.double(), 1e-6).numpy()
    tenth = Decimal(1) / Decimal(10)
    for i, p0 in enumerate(pos):
        s = float(_dec_pow(Decimal(1) + Decimal(int(p0) + 1) / Decimal(2048), tenth))
        assert np.array_equal(q[i], O.f64_to_bf16_bits(n[i] * s)), i
    # K is not scaled on full layers, and the full layer applies no rotation
    k = O.prepare_qk(x[:, :8], w, pos, "full", False)
    assert np.array_equal(k, O.f64_to_bf16_bits(n[:, :8]))


# ------------------------------------------------------------------ RoPE

def test_rope_relative_position_invariance():
    rng = np.random.default_rng(4)
    q = rng.standard_normal((6, 128))
    k = rng.standard_normal((6, 128))
    for m, n in [(0, 0), (5, 3), (100, 7000), (1000, 999999)]:
        base = np.sum(O.rope(q, m) * O.rope(k, n), axis=-1)
        for d in [1, 511, 99999, 1048575]:
            moved = np.sum(O.rope(q, m + d) * O.rope(k, n + d), axis=-1)
            np.testing.assert_allclose(moved, base, atol=1e-9, rtol=0)


def test_rope_identity_at_zero_and_norm_preserving():
    rng = np.random.default_rng(5)
    y = rng.standard_normal((7, 128))
    assert np.array_equal(O.rope(y, 0), y)
    np.testing.assert_allclose(np.linalg.norm(O.rope(y, 123457), axis=-1), np.linalg.norm(y, axis=-1), rtol=1e-13)


@pytest.mark.parametrize("i,freq", [(0, 1.0), (16, 0.1), (32, 0.01), (48, 0.001)])
def test_rope_frequencies_and_direction(i, freq):
    # theta = 1e4, D = 128: pair i turns at 10^(-4 * 2i/128) = 10^(-i/16) rad per token
    e = np.zeros(128)
    e[i] = 1.0
    pos = 37.0
    out = O.rope(e, pos)
    a = pos * freq
    assert abs(out[i] - math.cos(a)) < 1e-12 and abs(out[i + 64] - math.sin(a)) < 1e-12
    others = np.ones(128, dtype=bool)
    others[[i, i + 64]] = False
    assert np.all(out[others] == 0)
    e2 = np.zeros(128)
    e2[i + 64] = 1.0
    out2 = O.rope(e2, pos)
    assert abs(out2[i] + math.sin(a)) < 1e-12 and abs(out2[i + 64] - math.cos(a)) < 1e-12


# ------------------------------------------------------------------ attention core

def _dense_call(T, kind, seed, q_len=None, kv_dtype="bf16"):
    q_len = T if q_len is None else q_len
    return synth.make_call([q_len], [T], kind, kv_dtype, [seed, 77])


def test_attention_matches_sdpa_textbook_routine():
    """Full layer, no rotation, no SSMax, unit gate: causal SDPA with KV heads repeated
    (query head h reads KV head h // 6) and the default scale 1/sqrt(128)."""
    T = 150
    c = _dense_call(T, "full", 1)
    inp = c.oracle_inputs()
    seq, pos = O.new_token_positions(inp["q_start"], inp["kv_len"])
    # write raw k/v as the cache contents, use raw q as q'
    kc = O.store_kv(inp["k_cache"], inp["block_table"], seq, pos, inp["k"], "bf16")
    vc = O.store_kv(inp["v_cache"], inp["block_table"], seq, pos, inp["v"], "bf16")
    o = O.attention_rows(inp["q"], kc, vc, inp["block_table"], seq, pos, "full", "bf16")
    q = torch.from_numpy(O.bf16_bits_to_f64(inp["q"])).permute(1, 0, 2)
    k = torch.from_numpy(O.bf16_bits_to_f64(inp["k"])).permute(1, 0, 2).repeat_interleave(6, 0)
    v = torch.from_numpy(O.bf16_bits_to_f64(inp["v"])).permute(1, 0, 2).repeat_interleave(6, 0)
    ref = torch.nn.functional.scaled_dot_product_attention(q, k, v, is_causal=True)
    np.testing.assert_allclose(o, ref.permute(1, 0, 2).numpy(), atol=1e-12, rtol=0)
    # sliding layer: the same routine with a band mask of 512 keys (own token included)
    T = 700
    c = _dense_call(T, "swa", 2)
    inp = c.oracle_inputs()
    seq, pos = O.new_token_positions(inp["q_start"], inp["kv_len"])
    kc = O.store_kv(inp["k_cache"], inp["block_table"], seq, pos, inp["k"], "bf16")
    vc = O.store_kv(inp["v_cache"], inp["block_table"], seq, pos, inp["v"], "bf16")
    rows = np.array([0, 1, 255, 510, 511, 512, 513, 600, 699])
    o = O.attention_rows(inp["q"][rows], kc, vc, inp["block_table"], seq[rows], pos[rows], "swa", "bf16")
    i = torch.arange(T)[:, None]
    j = torch.arange(T)[None, :]
    band = (j <= i) & (j > i - 512)
    q = torch.from_numpy(O.bf16_bits_to_f64(inp["q"])).permute(1, 0, 2)
    k = torch.from_numpy(O.bf16_bits_to_f64(inp["k"])).permute(1, 0, 2).repeat_interleave(6, 0)
    v = torch.from_numpy(O.bf16_bits_to_f64(inp["v"])).permute(1, 0, 2).repeat_interleave(6, 0)
    ref = torch.nn.functional.scaled_dot_product_attention(q, k, v, attn_mask=band)
    np.testing.assert_allclose(o, ref.permute(1, 0, 2).numpy()[rows], atol=1e-12, rtol=0)


def test_window_equals_full_up_to_512_keys_and_differs_after():
    T = 513
    c = _dense_call(T, "full", 3)
    inp = c.oracle_inputs()
    seq, pos = O.new_token_positions(inp["q_start"], inp["kv_len"])
    kc = O.store_kv(inp["k_cache"], inp["block_table"], seq, pos, inp["k"], "bf16")
    vc = O.store_kv(inp["v_cache"], inp["block_table"], seq, pos, inp["v"], "bf16")
    of = O.attention_rows(inp["q"], kc, vc, inp["block_table"], seq, pos, "full", "bf16")
    ow = O.attention_rows(inp["q"], kc, vc, inp["block_table"], seq, pos, "swa", "bf16")
    assert np.array_equal(of[:512], ow[:512])          # T <= 512: identical, bitwise
    assert not np.allclose(of[512], ow[512], atol=1e-6)  # key 0 leaves the window at pos 512


def test_softmax_rows_sum_to_one_and_first_token_returns_v0():
    rng = np.random.default_rng(6)
    z = rng.standard_normal((50, 1000)) * 30
    p = O.softmax(z)
    assert np.all(p >= 0)
    np.testing.assert_allclose(p.sum(-1), 1.0, atol=1e-12)
    c = _dense_call(40, "full", 4)
    inp = c.oracle_inputs()
    seq, pos = O.new_token_positions(inp["q_start"], inp["kv_len"])
    kc = O.store_kv(inp["k_cache"], inp["block_table"], seq, pos, inp["k"], "bf16")
    vc = O.store_kv(inp["v_cache"], inp["block_table"], seq, pos, inp["v"], "bf16")
    o = O.attention_rows(inp["q"][:1], kc, vc, inp["block_table"], seq[:1], pos[:1], "full", "bf16")
    v0 = O.bf16_bits_to_f64(inp["v"][0])
    assert np.array_equal(o[0], np.repeat(v0, 6, axis=0))


def test_gate_bias_switches_heads_off_and_on():
    rng = np.random.default_rng(7)
    o = rng.standard_normal((5, 48, 128))
    gate = bits_bf16(torch.from_numpy(rng.standard_normal((5, 6144)).astype(np.float32)).bfloat16())
    bias = np.array([0.0] * 48)
    bias[3] = -1e4
    bias[7] = 1e4
    bias_bits = O.f64_to_bf16_bits(bias)
    y = O.head_gate(o, gate, bias_bits)
    assert np.all(y[:, 3, :] == 0.0)
    assert np.array_equal(y[:, 7, :], o[:, 7, :])
    g = O.bf16_bits_to_f64(gate).reshape(5, 48, 128)
    np.testing.assert_allclose(y[:, 0, :], o[:, 0, :] / (1 + np.exp(-g[:, 0, :])), rtol=1e-15)


def test_kv_size_closed_form_matches_pages():
    g = golden()
    m, kv = g["model"], g["kv_cache"]
    assert (O.NUM_Q_HEADS, O.NUM_KV_HEADS, O.HEAD_DIM, O.WINDOW, O.PAGE_SIZE) == (
        m["num_q_heads"], m["num_kv_heads"], m["head_dim"], m["window"], m["page_size"])
    assert O.NUM_FULL_LAYERS == m["num_full_layers"] and O.NUM_LAYERS == m["num_layers"]
    assert m["num_full_layers"] + m["num_swa_layers"] == m["num_layers"]
    assert O.kv_bytes_per_token(bytes_per_value=1) == kv["values_per_token"]
    assert O.kv_bytes_per_token(bytes_per_value=2) == kv["bytes_per_token_bf16"] == 36 * 1024
    assert O.kv_bytes_per_token(bytes_per_value=1) == kv["bytes_per_token_fp8"] == 18 * 1024
    ctx = m["context_limit"]
    assert O.kv_bytes_per_token(bytes_per_value=1) * ctx / 2 ** 30 == kv["fp8_gib_at_1m_tokens"]
    all_global = O.kv_bytes_per_token(num_full_layers=m["num_layers"], bytes_per_value=2)
    assert all_global == kv["bytes_per_token_if_all_52_layers_global_bf16"]
    assert all_global * ctx / 2 ** 30 == kv["bf16_gib_at_1m_if_all_global"]
    swa_windows = m["num_swa_layers"] * O.WINDOW * O.kv_bytes_per_token(1, bytes_per_value=2)
    total = (O.kv_bytes_per_token(bytes_per_value=2) * ctx + swa_windows) / 2 ** 30
    assert round(total, 2) == kv["bf16_gib_at_1m_incl_swa_windows"]


# ------------------------------------------------------------------ paging, fp8, composition

def test_page_permutation_does_not_change_results():
    a = synth.make_call([3, 70], [130, 70], "full", "bf16", [9, 1])
    inp = a.oracle_inputs()
    ra = O.layer_call(inp)
    # move every data page to a new physical index
    P = inp["k_cache"].shape[0]
    perm = np.random.default_rng(5).permutation(P)
    inv = np.argsort(perm)
    inp2 = dict(inp)
    inp2["k_cache"] = inp["k_cache"][inv]
    inp2["v_cache"] = inp["v_cache"][inv]
    inp2["block_table"] = perm[inp["block_table"]].astype(np.int32)
    rb = O.layer_call(inp2)
    assert np.array_equal(ra["y"], rb["y"])


def test_unvisited_slots_are_never_read():
    c = synth.make_call([4, 1], [600, 900], "swa", "bf16", [10, 0])
    inp = c.oracle_inputs()
    assert c.poison_page >= 0
    r = O.layer_call(inp)
    assert np.all(np.isfinite(r["y"]))


def test_fp8_store_roundtrip_error_bound():
    c = synth.make_call([16], [80], "full", "fp8", [12, 1])
    inp = c.oracle_inputs()
    seq, pos = O.new_token_positions(inp["q_start"], inp["kv_len"])
    vc = O.store_kv(inp["v_cache"], inp["block_table"], seq, pos, inp["v"], "fp8", inp["v_scale"])
    back = O.read_kv(vc, inp["block_table"], 0, pos, "fp8", inp["v_scale"])
    x = O.bf16_bits_to_f64(inp["v"])
    err = np.abs(back - x)
    # e4m3: relative spacing 2^-3 for normals (half of it after rounding), absolute
    # spacing 2^-9 * scale for subnormals; nothing here exceeds 448 * scale
    assert np.all(err <= np.maximum(np.abs(x) * 2 ** -4, 2 ** -10 * inp["v_scale"]) * (1 + 1e-12))


_E4M3_MAGS = [Fraction(m, 512) if e == 0 else Fraction(8 + m, 8) * Fraction(2) ** (e - 7)
              for e in range(16) for m in range(8) if not (e == 15 and m == 7)]


def _nearest_e4m3_exact(q: Fraction, negative: bool = False) -> int:
    """Code of the e4m3 value nearest to the exact rational q, ties to the even code,
    saturating at +-448; the sign bit is that of q, or `negative` when q is zero (-0). The 127 finite magnitudes are written from the format (exponent
    field e, mantissa m: (8 + m) 2^(e-10), or m 2^-9 when e = 0); the neighbours of |q|
    are found by bisection and compared in exact rational arithmetic."""
    import bisect

    a = min(abs(q), Fraction(448))
    hi = min(bisect.bisect_left(_E4M3_MAGS, a), len(_E4M3_MAGS) - 1)
    cands = [c for c in (hi - 1, hi) if c >= 0]
    best = min(cands, key=lambda c: (abs(_E4M3_MAGS[c] - a), c % 2))
    return best | (0x80 if (q < 0 or (q == 0 and negative)) else 0)


def test_fp8_store_is_nearest_e4m3_of_exact_quotient():
    """The stored code is the e4m3 value nearest to the exact quotient value/scale (the
    bf16 value and the fp32 scale taken as exact rationals): every finite bf16 pattern
    of magnitude below 8 is stored through store_kv at three scales and checked against
    an exact rational search. At the scales of the form amax/448 some quotients round
    in binary32 onto an e4m3 midpoint, so a single-precision quotient fails here."""
    allb = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    xv = O.bf16_bits_to_f64(allb)
    pats = allb[np.isfinite(xv) & (np.abs(xv) < 8)]
    n_tok = -(-len(pats) // (8 * 128))
    vals = np.zeros(n_tok * 8 * 128, dtype=np.uint16)
    vals[:len(pats)] = pats
    vals = vals.reshape(n_tok, 8, 128)
    cache = np.zeros((1, 8, 64, 128), dtype=np.uint8)
    bt = np.zeros((1, 1), dtype=np.int32)
    seq, pos = np.zeros(n_tok, dtype=np.int64), np.arange(n_tok)
    split = 0
    for scale in (float(np.float32(5.0625 / 448)), float(np.float32(4.9375 / 448)), 0.01018415205180645):
        out = O.store_kv(cache, bt, seq, pos, vals, "fp8", scale)[0][:, :n_tok, :]   # [8, n, 128]
        got = out.transpose(1, 0, 2).reshape(-1)[:len(pats)]
        s = Fraction(float(np.float32(scale)))
        for u, code in zip(pats, got):
            x = Fraction(struct.unpack("<f", struct.pack("<I", int(u) << 16))[0])
            want = _nearest_e4m3_exact(x / s, bool(u & 0x8000))
            assert code == want, (scale, hex(int(u)), int(code), want)
            q32 = Fraction(float(np.float32(float(x)) / np.float32(float(s))))
            split += _nearest_e4m3_exact(q32, bool(u & 0x8000)) != want
    assert split > 0   # binary32 quotients round some of these codes the other way


def test_bf16_round_of_f64_is_one_rounding():
    """bf16 rounding of fp64 values rounds once: values just off a bf16 midpoint (where
    going through binary32 first would land on the midpoint and round to even) round to
    the nearer side. Reference: integer rounding of the fp64 significand to 8 bits."""
    rng = np.random.default_rng(41)
    base = rng.integers(1 << 14, 0x7F00, 4000).astype(np.uint32) << 16   # finite bf16 values
    mid = (base | np.uint32(0x8000)).view(np.float32).astype(np.float64)   # bf16 midpoints
    x = np.concatenate([mid * (1 + 2.0 ** -40), mid * (1 - 2.0 ** -40), mid,
                        rng.standard_normal(20000) * 1e3])
    u = x.view(np.uint64)
    keep, low = u >> np.uint64(45), u & np.uint64((1 << 45) - 1)
    up = (low > np.uint64(1 << 44)) | ((low == np.uint64(1 << 44)) & ((keep & np.uint64(1)) == 1))
    ref = ((keep + up.astype(np.uint64)) << np.uint64(45)).view(np.float64)
    assert np.array_equal(O.bf16_round(x), ref)


def test_prepare_k_sliding_layer_is_norm_then_rotation_then_one_rounding():
    """Sliding layers: bf16 of RoPE(rms_norm(x)), checked bit for bit against torch's
    rms_norm followed by an independent rotation (each pair (i, i + 64) as the complex
    number y_i + i y_(i+64), multiplied by exp(i pos theta^(-2i/128))), rounded once by
    integer rounding of the fp64 significand. Non-uniform norm weights make rotating
    before the norm, or rounding between the two steps, fail the comparison."""
    rng = np.random.default_rng(31)
    x = bits_bf16(torch.from_numpy(rng.standard_normal((5, 8, 128)).astype(np.float32)).bfloat16())
    wt = (1 + 0.1 * torch.from_numpy(rng.standard_normal(128).astype(np.float32))).bfloat16()
    pos = np.array([0, 1, 511, 99999, 1048583])
    got = O.prepare_qk(x, bits_bf16(wt), pos, "swa", False)
    gq = O.prepare_qk(np.repeat(x, 6, axis=1), bits_bf16(wt), pos, "swa", True)
    n = torch.nn.functional.rms_norm(torch.from_numpy(O.bf16_bits_to_f64(x)), (128,), wt.double(), 1e-6)
    z = torch.complex(n[..., :64], n[..., 64:])
    inv_freq = 1.0 / (torch.tensor(1e4, dtype=torch.float64) ** (torch.arange(0, 128, 2, dtype=torch.float64) / 128))
    ang = torch.from_numpy(pos.astype(np.float64))[:, None] * inv_freq[None, :]
    rot = z * torch.polar(torch.ones_like(ang), ang)[:, None, :]
    y = torch.cat([rot.real, rot.imag], dim=-1).numpy()
    u = y.view(np.uint64)
    keep, low = u >> np.uint64(45), u & np.uint64((1 << 45) - 1)
    up = (low > np.uint64(1 << 44)) | ((low == np.uint64(1 << 44)) & ((keep & np.uint64(1)) == 1))
    r = ((keep + up.astype(np.uint64)) << np.uint64(45)).view(np.float64).astype(np.float32)
    ref = (r.view(np.uint32) >> np.uint32(16)).astype(np.uint16)
    assert np.array_equal(got, ref)
    # Q gets the same transform on sliding layers (no SSMax there)
    assert np.array_equal(gq, np.repeat(ref, 6, axis=1))


def test_block_is_causal_within_itself():
    c = synth.make_call([6], [200], "full", "bf16", [13, 1])
    inp = c.oracle_inputs()
    r1 = O.layer_call(inp)
    inp2 = dict(inp)
    k2 = inp["k"].copy()
    v2 = inp["v"].copy()
    k2[4:] ^= np.uint16(0x0040)
    v2[4:] ^= np.uint16(0x0040)
    inp2["k"], inp2["v"] = k2, v2
    r2 = O.layer_call(inp2)
    assert np.array_equal(r1["y"][:4], r2["y"][:4])
    assert not np.array_equal(r1["y"][4:], r2["y"][4:])


def test_decode_equals_last_row_of_prefill():
    for kind in ("full", "swa"):
        T = 600
        pre = synth.make_call([T], [T], kind, "bf16", [14, 3])
        inp = pre.oracle_inputs()
        rp = O.layer_call(inp)
        dec = dict(inp)
        # the first T-1 tokens are now cached (as the prefill stored them); one new token
        dec["k_cache"], dec["v_cache"] = rp["k_cache"], rp["v_cache"]
        dec["q_start"] = np.array([0, 1], dtype=np.int32)
        dec["kv_len"] = np.array([T], dtype=np.int32)
        for key in ("q", "k", "v", "gate"):
            dec[key] = inp[key][T - 1:]
        rd = O.layer_call(dec)
        assert np.array_equal(rd["y"][0], rp["y"][T - 1])


# ------------------------------------------------------------------ loop implementation

def _loop_layer(inp):
    """The whole layer written with Python loops and the math module only."""
    Hq, Hkv, D = 48, 8, 128
    G = Hq // Hkv

    def bf(bits):
        return struct.unpack("<f", struct.pack("<I", int(bits) << 16))[0]

    def rbf(x):
        # nearest bf16 value, ties to even, in exact rational arithmetic
        if x == 0:
            return 0.0
        _, e = math.frexp(abs(x))
        spacing = Fraction(2) ** (e - 1 - 7)
        return math.copysign(float(round(Fraction(abs(x)) / spacing) * spacing), x)

    q_start, kv_len, bt = inp["q_start"], inp["kv_len"], inp["block_table"]
    kind = inp["kind"]
    y_all = []
    keys = {}   # (b, pos) -> (k[Hkv][D], v[Hkv][D])
    # cached tokens straight from the pages
    toks = []
    for b in range(len(kv_len)):
        n = int(q_start[b + 1] - q_start[b])
        for i in range(n):
            toks.append((b, int(kv_len[b]) - n + i, int(q_start[b]) + i))
    newpos = {(b, p) for b, p, _ in toks}

    def cached(b, p):
        page = int(bt[b][p // 64])
        s = p % 64
        return ([[bf(inp["k_cache"][page, g, s, d]) for d in range(D)] for g in range(Hkv)],
                [[bf(inp["v_cache"][page, g, s, d]) for d in range(D)] for g in range(Hkv)])

    def prep(x, w, p, is_q):
        ms = sum(t * t for t in x) / D
        r = 1.0 / math.sqrt(ms + 1e-6)
        y = [w[d] * x[d] * r for d in range(D)]
        if kind == "swa":
            out = [0.0] * D
            for i in range(D // 2):
                a = p * 10000.0 ** (-2.0 * i / D)
                out[i] = y[i] * math.cos(a) - y[i + 64] * math.sin(a)
                out[i + 64] = y[i + 64] * math.cos(a) + y[i] * math.sin(a)
            y = out
        elif is_q:
            y = [t * (1.0 + (p + 1) / 2048.0) ** 0.1 for t in y]
        return [rbf(t) for t in y]

    wq = [bf(t) for t in inp["q_norm_w"]]
    wk = [bf(t) for t in inp["k_norm_w"]]
    for b, p, t in toks:
        keys[(b, p)] = ([prep([bf(x) for x in inp["k"][t, g]], wk, p, False) for g in range(Hkv)],
                        [[bf(x) for x in inp["v"][t, g]] for g in range(Hkv)])
    for b, p, t in toks:
        lo = 0 if kind == "full" else max(0, p - 511)
        kv = [keys[(b, j)] if (b, j) in newpos else cached(b, j) for j in range(lo, p + 1)]
        yt = []
        for h in range(Hq):
            qh = prep([bf(x) for x in inp["q"][t, h]], wq, p, True)
            g = h // G
            z = [sum(qh[d] * kvj[0][g][d] for d in range(D)) / math.sqrt(D) for kvj in kv]
            m = max(z)
            e = [math.exp(zz - m) for zz in z]
            s = sum(e)
            o = [sum(e[j] / s * kv[j][1][g][d] for j in range(len(kv))) for d in range(D)]
            bias = bf(inp["gate_bias"][h])
            yt.append([o[d] / (1.0 + math.exp(-(bf(inp["gate"][t, h * D + d]) + bias))) for d in range(D)])
        y_all.append(yt)
    return np.array(y_all)


@pytest.mark.parametrize("kind", ["full", "swa"])
def test_vectorised_oracle_equals_loop_implementation(kind):
    c = synth.make_call([3, 2], [5, 9], kind, "bf16", [15, 2])
    inp = c.oracle_inputs()
    r = O.layer_call(inp)
    ref = _loop_layer(inp)
    np.testing.assert_allclose(r["y"], ref, atol=1e-12, rtol=0)


def test_long_context_path_equals_short_path():
    c = synth.make_call([2, 1], [3000, 1500], "full", "fp8", [16, 1])
    inp = c.oracle_inputs()
    seq, pos = O.new_token_positions(inp["q_start"], inp["kv_len"])
    q = O.prepare_qk(inp["q"], inp["q_norm_w"], pos, "full", True)
    a = O.attention_rows(q, inp["k_cache"], inp["v_cache"], inp["block_table"], seq, pos - 5,
                         "full", "fp8", inp["k_scale"], inp["v_scale"])
    b = O.attention_rows_long(q, inp["k_cache"], inp["v_cache"], inp["block_table"], seq, pos - 5,
                              "full", "fp8", inp["k_scale"], inp["v_scale"], key_chunk=333)
    c2 = synth.make_call([3, 1], [900, 700], "swa", "bf16", [17, 0])
    inp = c2.oracle_inputs()
    seq, pos = O.new_token_positions(inp["q_start"], inp["kv_len"])
    q = O.prepare_qk(inp["q"], inp["q_norm_w"], pos, "swa", True)
    kc = O.store_kv(inp["k_cache"], inp["block_table"], seq, pos, inp["k"], "bf16")
    vc = O.store_kv(inp["v_cache"], inp["block_table"], seq, pos, inp["v"], "bf16")
    a2 = O.attention_rows(q, kc, vc, inp["block_table"], seq, pos, "swa", "bf16")
    b2 = O.attention_rows_long(q, kc, vc, inp["block_table"], seq, pos, "swa", "bf16", key_chunk=100)
    np.testing.assert_allclose(a2, b2, atol=1e-13, rtol=0)
    np.testing.assert_allclose(a, b, atol=1e-13, rtol=0)


# ------------------------------------------------------------------ projections

def _bits(t):
    return t.view(torch.int16).numpy().view(np.uint16)


def test_linear_equals_exact_rational_sum_on_small_shapes():
    """y[i, j] = sum_c x[i, c] W[j, c]: every term is an exact product of two bf16 values,
    summed here in exact rationals; the fp64 oracle may differ only by its own rounding."""
    x, w = synth.make_linear(3, 5, 64, [71, 0])
    y = O.linear(_bits(x), _bits(w))
    xf = [[Fraction(float(v)) for v in row] for row in x.float().numpy()]
    wf = [[Fraction(float(v)) for v in row] for row in w.float().numpy()]
    for i in range(3):
        for j in range(5):
            exact = sum(a * b for a, b in zip(xf[i], wf[j]))
            mass = sum(abs(a * b) for a, b in zip(xf[i], wf[j]))
            assert abs(Fraction(y[i, j]) - exact) <= mass * Fraction(64, 2 ** 53)


def test_linear_identity_permutation_and_row_sums():
    x, _ = synth.make_linear(4, 8, 64, [72, 0])
    one = torch.eye(64, dtype=torch.bfloat16)
    assert np.array_equal(O.linear(_bits(x), _bits(one)), x.double().numpy())
    perm = torch.from_numpy(np.random.default_rng(3).permutation(64))
    y = O.linear(_bits(x), _bits(one[perm]))
    assert np.array_equal(y, x.double().numpy()[:, perm.numpy()])          # column j is x[:, perm[j]]
    ones = torch.ones(1, 64, dtype=torch.bfloat16)
    np.testing.assert_allclose(O.linear(_bits(x), _bits(ones))[:, 0], x.double().numpy().sum(axis=1),
                               rtol=0, atol=1e-12)


def test_linear_orientation_is_x_times_w_transposed():
    """A transposed operand would fail on shapes where only x W^T is defined."""
    x, w = synth.make_linear(3, 7, 128, [73, 0])
    y = O.linear(_bits(x), _bits(w))
    assert y.shape == (3, 7)
    np.testing.assert_allclose(y, x.double().numpy() @ w.double().numpy().T, rtol=0, atol=1e-12)
