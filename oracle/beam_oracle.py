"""Plain fp64 CPU oracle for the hybrid sliding-window / NoPE GQA attention core.

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import, call or execute
this module: only the test suite, the smoke check and the CPU-baseline leg of the
benchmark use it. It shares no code with the HIP library and imports nothing from
it.

Sources (page title, then section):
  [P1] "SGLang natively supports Reflection's Beam" (LMSYS blog, Chinese text):
       Model architecture table; Hybrid attention and output gating; SSMax;
       Unified memory for target and draft KV; Fusion optimizations.
  [P2] "vLLM natively supports the Reflection Beam 501B MoE model" (Chinese text):
       Model architecture / Attention; Agent-driven optimization, changes 2 and 6.
  [P4] "Welcome Beam: a 501B open model" (Hugging Face launch summary, Chinese).
  [P5] "Reflection Beam 1.0 on vLLM: Day 0 Serving, Agent-Optimized Kernels, and
       DFlash2 Speculative Decoding": Attention: sliding-window layers plus NoPE
       full-attention layers; Agent-driven optimization made batch-1 decode 2.71x
       faster.

Everything is float64 except the rounding points the specification fixes: q' and
k' are rounded to bf16 after norm + rotation/scaling, and the stored K/V carry the
cache dtype (bf16, or fp8 e4m3 with a per-tensor fp32 scale). Inputs are the exact
bit patterns the GPU receives (uint16 for bf16, uint8 for fp8 codes).

Readings taken where the pages are silent (each is listed in the design notes):
  * RoPE is rotate-half over all 128 dims, 0-based positions, theta = 1e4; the
    angle is formed in fp64.
  * SSMax multiplies q only, after RMSNorm, by (1 + p/2048)^0.1 with p = pos + 1.
  * One [128] RMSNorm weight for Q and one for K, shared across heads (a per-head
    [H,128] weight is also accepted); eps = 1e-6; y = w * x / sqrt(mean(x^2) + eps).
  * The window holds 512 keys including the query's own token: [pos-511, pos].
  * Query head h reads KV head floor(h / (Hq/Hkv)).
  * gate column h*128 + d; per-head bias broadcast over d; V is not normalised.
  * New tokens in one call see earlier new tokens and themselves (causal block).
  * fp8 is OCP E4M3FN with saturating round-to-nearest-even; stored = e4m3(k'/scale),
    the quotient value/scale formed in fp64. A bf16 value over an fp32 scale is never
    within 2^-53 (relative) of an e4m3 rounding midpoint without lying on it, so this
    code is the nearest e4m3 value to the exact quotient.

Parity status: every function below is pinned by the CPU test-suite against closed
forms, library routines or invariants. The readings above that no page fixes are pinned
to the open implementations of the same components in the `transformers` library:
the window and causal masks (masking_utils), the query-head -> KV-head mapping
(Llama's repeat_kv), the rotary pairing, direction and frequencies (Llama's rotary
embedding) and the per-head norm with one [head_dim] weight (Qwen3's q_norm). The fp8
scale choice (per tensor, amax/448) is a property of the generated inputs; the oracle
takes the scale as given ("parity unpinned" for that choice only).
"""

from __future__ import annotations

import math

import numpy as np

# Model constants [P5, Attention: sliding-window layers plus NoPE full-attention
# layers]; [P1, Model architecture table].
NUM_Q_HEADS = 48
NUM_KV_HEADS = 8
HEAD_DIM = 128
WINDOW = 512
PAGE_SIZE = 64  # 64-token pages (SGLang launch flags in [P1], appendix)
NUM_FULL_LAYERS = 9
NUM_LAYERS = 52
# Constants the pages leave open, fixed by the specification of this library.
ROPE_THETA = 1.0e4
RMS_EPS = 1.0e-6
SSMAX_BASE = 2048.0
SSMAX_EXPONENT = 0.1
SM_SCALE = 1.0 / math.sqrt(128.0)

KIND_SWA = "swa"
KIND_FULL = "full"


# ----------------------------------------------------------------------------------
# Storage formats
# ----------------------------------------------------------------------------------

def bf16_bits_to_f64(bits) -> np.ndarray:
    """Value of bf16 bit patterns: a bf16 is the upper half of an IEEE binary32."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    with np.errstate(invalid="ignore"):
        return b.view(np.float32).astype(np.float64)


def bf16_round(x) -> np.ndarray:
    """Round float64 values to the nearest bf16 value, ties to even (IEEE RNE).

    bf16 keeps 8 significant bits (1 implicit + 7 stored) and binary32's exponent
    range. For |x| in [2^e, 2^(e+1)) the spacing is 2^(e-7); below 2^-126 the
    spacing is fixed at 2^-133 (subnormals). Values past the largest finite bf16
    (by half a spacing or more) become +-inf.
    """
    x = np.asarray(x, dtype=np.float64)
    out = np.array(x, copy=True)
    fin = np.isfinite(x) & (x != 0)
    ax = np.abs(x[fin])
    _, e2 = np.frexp(ax)            # ax = m * 2^e2, m in [0.5, 1)
    e = e2.astype(np.int64) - 1     # ax in [2^e, 2^(e+1))
    e = np.maximum(e, -126)
    spacing = np.ldexp(1.0, (e - 7).astype(np.int64))
    r = np.rint(ax / spacing) * spacing   # np.rint rounds half to even
    max_bf16 = (2.0 - 2.0 ** -7) * 2.0 ** 127
    r = np.where(r > max_bf16, np.inf, r)
    out[fin] = np.copysign(r, x[fin])
    return out


def f64_to_bf16_bits(x) -> np.ndarray:
    """bf16 bit patterns of float64 values (rounded to nearest even)."""
    r = bf16_round(x).astype(np.float32)  # exact: every bf16 value is a binary32 value
    return (r.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def _e4m3_formula(codes) -> np.ndarray:
    """Value of OCP FP8 E4M3FN codes: sign, 4 exponent bits (bias 7), 3 mantissa bits.

    Exponent field 0 holds subnormals M/8 * 2^-6; S.1111.111 is NaN; there is no inf.
    """
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    s = np.where((c >> 7) & 1, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    val = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * np.ldexp(1.0, e - 7))
    val = s * val
    return np.where((e == 15) & ((c & 7) == 7), np.nan, val)


# the value of every one of the 256 codes, from the formula above
_E4M3_ALL_VALUES = _e4m3_formula(np.arange(256, dtype=np.uint8))


def e4m3_to_f64(codes) -> np.ndarray:
    """Value of OCP FP8 E4M3FN codes (the formula above, looked up per code)."""
    return _E4M3_ALL_VALUES[np.asarray(codes, dtype=np.uint8)]


_E4M3_POS_CODES = np.arange(0, 0x7F, dtype=np.uint8)          # +0 .. +448, NaN excluded
_E4M3_POS_VALUES = e4m3_to_f64(_E4M3_POS_CODES)               # strictly increasing
E4M3_MAX = float(_E4M3_POS_VALUES[-1])                        # 448


def f64_to_e4m3(x) -> np.ndarray:
    """Encode float64 values as OCP E4M3FN codes: saturate to +-448, then round to the
    nearest representable value with ties to the even code (even mantissa). NaN -> 0x7F.
    """
    x = np.asarray(x, dtype=np.float64)
    ax = np.minimum(np.abs(x), E4M3_MAX)
    ax = np.where(np.isnan(ax), 0.0, ax)
    vals = _E4M3_POS_VALUES
    hi = np.clip(np.searchsorted(vals, ax, side="left"), 0, len(vals) - 1)
    lo = np.clip(hi - 1, 0, len(vals) - 1)
    d_hi = vals[hi] - ax
    d_lo = ax - vals[lo]
    pick_lo = (d_lo < d_hi) | ((d_lo == d_hi) & (lo % 2 == 0))
    mag = np.where(pick_lo, lo, hi).astype(np.uint8)
    sign = np.where(np.signbit(x), np.uint8(0x80), np.uint8(0))
    code = (mag | sign).astype(np.uint8)
    return np.where(np.isnan(x), np.uint8(0x7F), code).astype(np.uint8)


# ----------------------------------------------------------------------------------
# Per-head Q/K transforms
# [P5, Attention: ...]: Q and K are RMS-normalised per head before RoPE or SSMax.
# [P4]: norm, RoPE and query scaling are fp32 steps of the model; the oracle keeps
# fp64 and rounds to bf16 once, after them.
# ----------------------------------------------------------------------------------

def rms_norm(x, w, eps: float = RMS_EPS) -> np.ndarray:
    """y = w * x / sqrt(mean(x^2) + eps) over the last axis (one head of 128 values)."""
    x = np.asarray(x, dtype=np.float64)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return np.asarray(w, dtype=np.float64) * x / np.sqrt(ms + eps)


def ssmax_scale(p, base: float = SSMAX_BASE, exponent: float = SSMAX_EXPONENT):
    """SSMax query scale for 1-based position p: (1 + p/base)^exponent.

    [P5, Attention: ...] and [P2, Attention] give the 1-based form (1 + p/2048)^0.1;
    [P1, SSMax] writes the same with a zero-based position p0 as (1 + (p0+1)/2048).
    """
    p = np.asarray(p, dtype=np.float64)
    return np.power(1.0 + p / base, exponent)


def rope_inv_freq(head_dim: int = HEAD_DIM, theta: float = ROPE_THETA) -> np.ndarray:
    """Rotation frequency of pair i (i < head_dim/2): theta^(-2i/head_dim)."""
    i = np.arange(head_dim // 2, dtype=np.float64)
    return np.power(theta, -2.0 * i / head_dim)


def rope(y, pos, theta: float = ROPE_THETA) -> np.ndarray:
    """Rotate-half RoPE at 0-based positions `pos` (sliding-window layers only,
    [P5, Attention: ...]). y: [..., D], pos broadcast over the leading axes.

    Pair (i, i + D/2) turns by angle pos * theta^(-2i/D):
      y'_i       = y_i cos(a) - y_{i+D/2} sin(a)
      y'_{i+D/2} = y_{i+D/2} cos(a) + y_i sin(a)
    """
    y = np.asarray(y, dtype=np.float64)
    half = y.shape[-1] // 2
    ang = np.asarray(pos, dtype=np.float64)[..., None] * rope_inv_freq(y.shape[-1], theta)
    c, s = np.cos(ang), np.sin(ang)
    a, b = y[..., :half], y[..., half:]
    return np.concatenate([a * c - b * s, b * c + a * s], axis=-1)


def prepare_qk(x_bits, w_bits, pos, kind: str, is_query: bool, *,
               theta: float = ROPE_THETA, eps: float = RMS_EPS,
               ssmax_base: float = SSMAX_BASE, ssmax_exponent: float = SSMAX_EXPONENT):
    """One fused step of [P2, Agent-driven optimization, change 2]: per-head RMSNorm,
    then RoPE (sliding-window layer, Q and K) or SSMax (full NoPE layer, Q only),
    then one bf16 rounding. x_bits: [N, H, D] bf16 bits; pos: [N] 0-based.
    w_bits: [D] (shared by heads) or [H, D]. Returns bf16 bits [N, H, D].
    """
    x = bf16_bits_to_f64(x_bits)
    w = bf16_bits_to_f64(w_bits)
    if w.ndim == 1:
        w = w[None, None, :]
    else:
        w = w[None, :, :]
    y = rms_norm(x, w, eps)
    pos = np.asarray(pos, dtype=np.int64)
    if kind == KIND_SWA:
        y = rope(y, pos[:, None], theta)
    elif kind == KIND_FULL:
        if is_query:
            y = y * ssmax_scale(pos + 1, ssmax_base, ssmax_exponent)[:, None, None]
    else:
        raise ValueError(kind)
    return f64_to_bf16_bits(y)


# ----------------------------------------------------------------------------------
# Paged KV cache: one virtual->physical contract for reads and writes
# [P1, Unified memory for target and draft KV]; 64-token pages.
# Cache arrays: [num_pages, Hkv, PAGE, D] of bf16 bits (uint16) or fp8 codes (uint8).
# ----------------------------------------------------------------------------------

def new_token_positions(q_start, kv_len):
    """For each new token (in call order): its sequence index and 0-based position.
    Sequence b owns tokens q_start[b]..q_start[b+1]-1; kv_len[b] counts the keys after
    the call, new ones included, so the i-th new token sits at kv_len[b] - n_b + i.
    """
    q_start = np.asarray(q_start, dtype=np.int64)
    kv_len = np.asarray(kv_len, dtype=np.int64)
    seq, pos = [], []
    for b in range(len(kv_len)):
        n = q_start[b + 1] - q_start[b]
        seq.extend([b] * n)
        pos.extend(range(kv_len[b] - n, kv_len[b]))
    return np.asarray(seq, dtype=np.int64), np.asarray(pos, dtype=np.int64)


def physical_slot(block_table, b, pos, page_size: int = PAGE_SIZE):
    """(physical page, slot within page) of token `pos` of sequence `b`."""
    pos = np.asarray(pos, dtype=np.int64)
    page = np.asarray(block_table, dtype=np.int64)[b, pos // page_size]
    return page, pos % page_size


def store_kv(cache, block_table, seq, pos, values_bits, kv_dtype: str, scale: float = 1.0):
    """Write new K (or V) rows into a copy of `cache` at their physical slots.
    values_bits: [N, Hkv, D] bf16 bits (k' after norm/rotation, or raw v).
    bf16 cache stores the bits unchanged; fp8 cache stores e4m3(value / scale), the
    quotient of the bf16 value and the fp32 scale formed in fp64 and rounded once to
    e4m3 (saturating, ties to even).
    """
    out = np.array(cache, copy=True)
    page, slot = physical_slot(block_table, seq, pos)
    if kv_dtype == "bf16":
        out[page, :, slot, :] = np.asarray(values_bits, dtype=np.uint16)
    elif kv_dtype == "fp8":
        quotient = bf16_bits_to_f64(values_bits) / float(np.float32(scale))
        out[page, :, slot, :] = f64_to_e4m3(quotient)
    else:
        raise ValueError(kv_dtype)
    return out


def read_kv(cache, block_table, b: int, positions, kv_dtype: str, scale: float = 1.0):
    """Dequantised fp64 K (or V) rows [len(positions), Hkv, D] of sequence b."""
    page, slot = physical_slot(block_table, b, positions)
    raw = np.asarray(cache)[page, :, slot, :]
    if kv_dtype == "bf16":
        return bf16_bits_to_f64(raw)
    if kv_dtype == "fp8":
        return e4m3_to_f64(raw) * float(scale)
    raise ValueError(kv_dtype)


# ----------------------------------------------------------------------------------
# Attention (plain definition: enumerate the visible keys, two-pass softmax)
# ----------------------------------------------------------------------------------

def visible_range(pos: int, kind: str, window: int = WINDOW):
    """Keys visible to the query at 0-based position `pos`: [lo, pos] inclusive.
    Full layer: all earlier keys and itself. Sliding layer: the most recent `window`
    keys, the query's own token included ([P5, Attention: ...])."""
    if kind == KIND_FULL:
        return 0, int(pos)
    if kind == KIND_SWA:
        return max(0, int(pos) - window + 1), int(pos)
    raise ValueError(kind)


def softmax(z, axis=-1):
    """Two-pass softmax: subtract the maximum, exponentiate, divide by the sum."""
    z = np.asarray(z, dtype=np.float64)
    m = np.max(z, axis=axis, keepdims=True)
    e = np.exp(z - m)
    return e / np.sum(e, axis=axis, keepdims=True)


def attend(q_hat, k, v, sm_scale: float = SM_SCALE):
    """Attention of query rows over one shared set of keys.
    q_hat: [R, Hq, D]; k, v: [L, Hkv, D] fp64. Query head h reads KV head h // G.
    Returns o [R, Hq, D] fp64 (not rounded)."""
    R, Hq, D = q_hat.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    o = np.empty((R, Hq, D), dtype=np.float64)
    for h in range(Hq):
        g = h // G
        z = sm_scale * (q_hat[:, h, :] @ k[:, g, :].T)       # [R, L]
        o[:, h, :] = softmax(z, axis=-1) @ v[:, g, :]
    return o


def attention_rows(q_bits, k_cache, v_cache, block_table, seq, pos, kind: str,
                   kv_dtype: str, k_scale: float = 1.0, v_scale: float = 1.0,
                   sm_scale: float = SM_SCALE, window: int = WINDOW):
    """Attention output o [R, Hq, D] (fp64) for query rows given by (seq[r], pos[r]).
    q_bits: [R, Hq, D] bf16 bits of q' (already normed and rotated/scaled). Each row
    reads exactly its visible keys from the paged cache; nothing else is touched.
    """
    q_hat = bf16_bits_to_f64(q_bits)
    R, Hq, D = q_hat.shape
    o = np.empty((R, Hq, D), dtype=np.float64)
    for r in range(R):
        lo, hi = visible_range(int(pos[r]), kind, window)
        keys = np.arange(lo, hi + 1)
        k = read_kv(k_cache, block_table, int(seq[r]), keys, kv_dtype, k_scale)
        v = read_kv(v_cache, block_table, int(seq[r]), keys, kv_dtype, v_scale)
        o[r] = attend(q_hat[r:r + 1], k, v, sm_scale)[0]
    return o


def attention_rows_long(q_bits, k_cache, v_cache, block_table, seq, pos, kind: str,
                        kv_dtype: str, k_scale: float = 1.0, v_scale: float = 1.0,
                        sm_scale: float = SM_SCALE, window: int = WINDOW,
                        key_chunk: int = 1 << 16):
    """Same result as attention_rows, for rows over very long contexts.

    Rows of one sequence are taken together; their keys are read one chunk at a time
    and each row's softmax is done in the textbook two passes: first the maximum of its
    visible scores, then exp(z - max), their sum and the weighted sum of V. Keys outside
    a row's visible range get weight exactly 0.
    """
    q_hat = bf16_bits_to_f64(q_bits)
    R, Hq, D = q_hat.shape
    Hkv = np.asarray(k_cache).shape[1]
    G = Hq // Hkv
    o = np.empty((R, Hq, D), dtype=np.float64)
    seq = np.asarray(seq, dtype=np.int64)
    pos = np.asarray(pos, dtype=np.int64)
    for b in np.unique(seq):
        rows = np.nonzero(seq == b)[0]
        lo_r = np.array([visible_range(int(pos[r]), kind, window)[0] for r in rows])
        hi_r = pos[rows]
        qb = q_hat[rows].reshape(len(rows), Hkv, G, D)                  # [r, g, G, D]
        m = np.full((len(rows), Hkv, G), -np.inf)
        chunks = range(int(lo_r.min()), int(hi_r.max()) + 1, key_chunk)

        def scores(s0):
            keys = np.arange(s0, min(int(hi_r.max()) + 1, s0 + key_chunk))
            kk = read_kv(k_cache, block_table, int(b), keys, kv_dtype, k_scale)   # [n, g, D]
            z = sm_scale * np.matmul(qb, kk.transpose(1, 2, 0)[None])          # [r, g, G, n]
            vis = (keys[None, :] >= lo_r[:, None]) & (keys[None, :] <= hi_r[:, None])
            return keys, np.where(vis[:, None, None, :], z, -np.inf)

        for s0 in chunks:                                   # pass 1: row maxima
            _, z = scores(s0)
            m = np.maximum(m, z.max(axis=-1))
        ssum = np.zeros_like(m)
        acc = np.zeros((len(rows), Hkv, G, D))
        for s0 in chunks:                                   # pass 2: weights, sums, PV
            keys, z = scores(s0)
            e = np.exp(z - m[..., None])
            ssum += e.sum(axis=-1)
            vv = read_kv(v_cache, block_table, int(b), keys, kv_dtype, v_scale)
            acc += np.matmul(e, vv.transpose(1, 0, 2)[None])                    # [r, g, G, D]
        o[rows] = (acc / ssum[..., None]).reshape(len(rows), Hq, D)
    return o


# ----------------------------------------------------------------------------------
# Output gate [P5, Attention: ...]: each head's output times sigmoid(gate + bias_h).
# ----------------------------------------------------------------------------------

def sigmoid(x):
    """1 / (1 + exp(-x)); exactly 0 where exp(-x) overflows to inf."""
    x = np.asarray(x, dtype=np.float64)
    with np.errstate(over="ignore"):
        return 1.0 / (1.0 + np.exp(-x))


def head_gate(o, gate_bits, bias_bits):
    """y[t, h, d] = o[t, h, d] * sigmoid(gate[t, h*D + d] + bias[h]).
    o: [N, Hq, D] fp64; gate_bits: [N, Hq*D] bf16 bits; bias_bits: [Hq] bf16 bits."""
    o = np.asarray(o, dtype=np.float64)
    N, Hq, D = o.shape
    gate = bf16_bits_to_f64(gate_bits).reshape(N, Hq, D)
    bias = bf16_bits_to_f64(bias_bits).reshape(1, Hq, 1)
    return o * sigmoid(gate + bias)


# ----------------------------------------------------------------------------------
# Projections on either side of the core ([P5] Attention: the gate has its own
# full-width projection; [P2] Agent-driven optimization: one packed GEMM feeds the fused
# norm kernel; o_proj after the gate)
# ----------------------------------------------------------------------------------

def linear(x_bits, w_bits) -> np.ndarray:
    """y = x W^T in fp64 from bf16 inputs: x [m, k], W [n, k] (the weight in its [out][in]
    layout), so y[i, j] = sum_c x[i, c] * W[j, c]. The packed projection maps the 5120
    hidden values to 6144 q + 1024 k + 1024 v + 6144 gate columns; o_proj maps the 6144
    gated attention values back to 5120. Exact products and an fp64 sum; no rounding."""
    return np.matmul(bf16_bits_to_f64(x_bits), bf16_bits_to_f64(w_bits).T)


# ----------------------------------------------------------------------------------
# KV-cache size closed form [P2, Attention] / [P5, Attention: ...] / [P4]
# ----------------------------------------------------------------------------------

def kv_bytes_per_token(num_full_layers: int = NUM_FULL_LAYERS, num_kv_heads: int = NUM_KV_HEADS,
                       head_dim: int = HEAD_DIM, bytes_per_value: int = 2) -> int:
    """Bytes of KV cache that grow with each token: only the full layers keep the
    whole history; each keeps K and V for every KV head."""
    return num_full_layers * 2 * num_kv_heads * head_dim * bytes_per_value


# ----------------------------------------------------------------------------------
# One layer call, composed from the steps above
# ----------------------------------------------------------------------------------

def layer_call(inp: dict, rows=None):
    """Run one attention-layer call the way the library's entry points chain:
    fused Q/K prepare + KV store, then attention over the paged cache, then the gate.

    inp keys: kind, kv_dtype, q_start [B+1], kv_len [B], block_table [B, P],
      q [N,Hq,D] / k [N,Hkv,D] / v [N,Hkv,D] / gate [N,Hq*D] bf16 bits,
      q_norm_w, k_norm_w [D] bf16 bits, gate_bias [Hq] bf16 bits,
      k_cache, v_cache (bits/codes), k_scale, v_scale; optional layer constants
      window, rope_theta, rms_eps, ssmax_base, ssmax_exponent, sm_scale (the model's
      values by default).
    rows: optional indices of new tokens whose attention output to compute (all if
      None). Returns dict with q_out bits [N,Hq,D], k_cache, v_cache (after the
      store), o [R,Hq,D] fp64 (ungated), y [R,Hq,D] fp64 (gated), rows.
    """
    kind, kv_dtype = inp["kind"], inp["kv_dtype"]
    seq, pos = new_token_positions(inp["q_start"], inp["kv_len"])
    consts = {"theta": float(inp.get("rope_theta", ROPE_THETA)),
              "eps": float(inp.get("rms_eps", RMS_EPS)),
              "ssmax_base": float(inp.get("ssmax_base", SSMAX_BASE)),
              "ssmax_exponent": float(inp.get("ssmax_exponent", SSMAX_EXPONENT))}
    q_out = prepare_qk(inp["q"], inp["q_norm_w"], pos, kind, True, **consts)
    k_out = prepare_qk(inp["k"], inp["k_norm_w"], pos, kind, False, **consts)
    k_cache = store_kv(inp["k_cache"], inp["block_table"], seq, pos, k_out, kv_dtype,
                       inp.get("k_scale", 1.0))
    v_cache = store_kv(inp["v_cache"], inp["block_table"], seq, pos, inp["v"], kv_dtype,
                       inp.get("v_scale", 1.0))
    if rows is None:
        rows = np.arange(len(pos))
    rows = np.asarray(rows, dtype=np.int64)
    fn = attention_rows_long if int(np.max(np.asarray(inp["kv_len"]))) > 65536 else attention_rows
    o = fn(q_out[rows], k_cache, v_cache, inp["block_table"], seq[rows], pos[rows], kind,
           kv_dtype, inp.get("k_scale", 1.0), inp.get("v_scale", 1.0),
           sm_scale=float(inp.get("sm_scale", SM_SCALE)), window=int(inp.get("window", WINDOW)))
    y = head_gate(o, np.asarray(inp["gate"])[rows], inp["gate_bias"])
    return {"q_out": q_out, "k_out": k_out, "k_cache": k_cache, "v_cache": v_cache,
            "o": o, "y": y, "rows": rows, "seq": seq, "pos": pos}
