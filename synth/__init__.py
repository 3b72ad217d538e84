"""Seeded synthetic inputs for one attention-layer call of the hybrid SWA / NoPE model.

This module draws random numbers, casts them to the storage dtypes with torch's
own casts, and lays out paged caches and page tables. It holds none of the
method's arithmetic (no norm, rotation, scaling, softmax or gate), so the oracle
and the HIP path can both be fed from it without sharing any of the method.

Value distributions follow the workload descriptions: q, k, v and gate N(0,1) in
bf16; Q/K norm weights 1 + 0.1 N(0,1) in bf16; per-head gate bias N(0,1) in bf16;
cached K/V N(0,1) ("already normed and rotated"), stored in bf16, or as fp8 e4m3
codes with a per-tensor fp32 scale amax/448 for fp8 caches. Physical pages are a
seeded random permutation of the pool. Slots that no call has written yet (the new
tokens' slots and the tail of each last page) hold NaN, and in sliding-window
layers every logical page wholly before the window points at one shared page of
NaN, so that any read outside the visible keys shows up in the results.
"""

from __future__ import annotations

import math
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np
import torch

HQ, HKV, D, PAGE = 48, 8, 128, 64
WINDOW = 512
BF16_NAN = 0x7FC0
FP8_NAN = 0x7F
_CHUNK = 1 << 22
_THREADS = min(16, max(1, (torch.get_num_threads() or 8)))


def _normal_f32(n: int, key) -> np.ndarray:
    """n standard normals (float32), filled chunk by chunk from generators seeded by
    (key..., chunk index) so the result does not depend on the thread count."""
    out = np.empty(n, dtype=np.float32)
    nchunks = (n + _CHUNK - 1) // _CHUNK

    def fill(i):
        s, e = i * _CHUNK, min(n, (i + 1) * _CHUNK)
        out[s:e] = np.random.default_rng(list(key) + [i]).standard_normal(e - s, dtype=np.float32)

    if nchunks <= 1:
        if n:
            fill(0)
    else:
        with ThreadPoolExecutor(_THREADS) as ex:
            list(ex.map(fill, range(nchunks)))
    return out


def _bf16(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(a).to(torch.bfloat16)


@dataclass
class LayerCall:
    """Inputs of one layer call. Tensors are CPU torch tensors; index arrays numpy."""
    name: str
    kind: str                      # "swa" | "full"
    kv_dtype: str                  # "bf16" | "fp8"
    q_start: np.ndarray            # int32 [B+1]
    kv_len: np.ndarray             # int32 [B], keys after this call (new ones included)
    block_table: np.ndarray        # int32 [B, max_pages]
    q: torch.Tensor                # bf16 [N, Hq, 128] (Hq = 48 unless heads is given)
    k: torch.Tensor                # bf16 [N, Hkv, 128] (Hkv = 8 unless heads is given)
    v: torch.Tensor                # bf16 [N, Hkv, 128]
    gate: torch.Tensor             # bf16 [N, Hq * 128]
    q_norm_w: torch.Tensor         # bf16 [128]
    k_norm_w: torch.Tensor         # bf16 [128]
    gate_bias: torch.Tensor        # bf16 [Hq]
    k_cache: torch.Tensor          # bf16 or uint8 [num_pages, Hkv, 64, 128]
    v_cache: torch.Tensor
    k_scale: float = 1.0
    v_scale: float = 1.0
    poison_page: int = -1
    extra: dict = field(default_factory=dict)

    @property
    def num_q_heads(self) -> int:
        return int(self.q.shape[1])

    @property
    def num_kv_heads(self) -> int:
        return int(self.k.shape[1])

    @property
    def num_seqs(self) -> int:
        return len(self.kv_len)

    @property
    def num_tokens(self) -> int:
        return int(self.q_start[-1])

    @property
    def q_lens(self) -> np.ndarray:
        return np.diff(self.q_start).astype(np.int64)

    @property
    def max_q_len(self) -> int:
        return int(self.q_lens.max()) if len(self.kv_len) else 0

    @property
    def max_kv_len(self) -> int:
        return int(np.max(self.kv_len)) if len(self.kv_len) else 0

    def oracle_inputs(self) -> dict:
        """Bit patterns as numpy arrays, in the oracle's layer_call format."""
        def bits(t):
            if t.dtype == torch.bfloat16:
                return t.view(torch.int16).numpy().view(np.uint16)
            return t.numpy()
        return {
            "kind": self.kind, "kv_dtype": self.kv_dtype,
            "q_start": self.q_start, "kv_len": self.kv_len, "block_table": self.block_table,
            "q": bits(self.q), "k": bits(self.k), "v": bits(self.v), "gate": bits(self.gate),
            "q_norm_w": bits(self.q_norm_w), "k_norm_w": bits(self.k_norm_w),
            "gate_bias": bits(self.gate_bias),
            "k_cache": bits(self.k_cache), "v_cache": bits(self.v_cache),
            "k_scale": self.k_scale, "v_scale": self.v_scale,
        }


def make_call(q_lens, kv_lens, kind: str, kv_dtype: str, seed, name: str = "case",
              spare_pages: int = 3, window: int = WINDOW, cache_device=None,
              fp8_scales=None, heads=None) -> LayerCall:
    """A layer call with the given new-token counts and total key counts per sequence.

    Draw order: page permutation, q, k, v, gate, q_norm_w, k_norm_w, gate_bias,
    cached K, cached V (each from its own seeded stream). With cache_device set (e.g.
    "cuda"), the cached K/V are drawn on that device by torch's seeded Philox generator
    instead of numpy (same distributions, different values, much faster for the
    multi-GiB caches); everything else is unchanged. The returned caches then live on
    that device. fp8_scales = (k_scale, v_scale) fixes the fp8 scales instead of
    amax / 448 of the drawn cache (so that several calls can share one cache descriptor).
    heads = (Hq, Hkv) replaces the 48 query and 8 KV heads, e.g. (6, 1) for the share of
    one of 8 GPUs that split the heads.
    """
    hq, hkv = (HQ, HKV) if heads is None else (int(heads[0]), int(heads[1]))
    assert hq > 0 and hkv > 0 and hq % hkv == 0
    q_lens = np.asarray(q_lens, dtype=np.int64)
    kv_lens = np.asarray(kv_lens, dtype=np.int64)
    assert np.all(q_lens >= 0) and np.all(kv_lens >= q_lens)
    B = len(q_lens)
    key = [int(s) for s in (seed if isinstance(seed, (list, tuple)) else [seed])]
    pages_per_seq = [(int(L) + PAGE - 1) // PAGE for L in kv_lens]
    max_pages = max(1, max(pages_per_seq) if B else 1)

    # Which logical pages hold data: all of them in a full layer; in a sliding layer
    # only those that overlap some new token's window (the rest share a NaN page).
    needed = []
    for b in range(B):
        first_pos = int(kv_lens[b] - q_lens[b])
        lo = max(0, first_pos - window + 1) if kind == "swa" else 0
        needed.append(list(range(lo // PAGE, pages_per_seq[b])) if pages_per_seq[b] else [])
    n_data = sum(len(x) for x in needed)
    has_poison = kind == "swa" and any(len(needed[b]) < pages_per_seq[b] for b in range(B))
    num_pages = n_data + spare_pages + (1 if has_poison else 0)
    perm = np.random.default_rng(key + [1]).permutation(num_pages).astype(np.int32)
    block_table = np.zeros((B, max_pages), dtype=np.int32)
    poison = int(perm[-1]) if has_poison else -1
    cursor = 0
    for b in range(B):
        block_table[b, :] = poison if has_poison else 0
        for j in needed[b]:
            block_table[b, j] = perm[cursor]
            cursor += 1

    N = int(q_lens.sum())
    q = _bf16(_normal_f32(N * hq * D, key + [2])).view(N, hq, D)
    k = _bf16(_normal_f32(N * hkv * D, key + [3])).view(N, hkv, D)
    v = _bf16(_normal_f32(N * hkv * D, key + [4])).view(N, hkv, D)
    gate = _bf16(_normal_f32(N * hq * D, key + [5])).view(N, hq * D)
    q_norm_w = _bf16(1.0 + 0.1 * _normal_f32(D, key + [6]))
    k_norm_w = _bf16(1.0 + 0.1 * _normal_f32(D, key + [7]))
    gate_bias = _bf16(_normal_f32(hq, key + [8]))

    # Cached K/V: N(0,1) values at every slot of every page, then NaN at the slots
    # that hold no cached token yet (new tokens' slots, tails, the shared NaN page).
    shape = (num_pages, hkv, PAGE, D)
    n_cache = num_pages * hkv * PAGE * D
    if cache_device is None:
        kc = _normal_bf16(n_cache, key + [9]).view(shape)
        vc = _normal_bf16(n_cache, key + [10]).view(shape)
    else:
        kc = _normal_bf16_device(n_cache, key + [9], cache_device).view(shape)
        vc = _normal_bf16_device(n_cache, key + [10], cache_device).view(shape)
    un_p, un_s = [], []
    for b in range(B):
        cached = int(kv_lens[b] - q_lens[b])
        for j in needed[b]:
            first = max(cached - j * PAGE, 0)
            if first < PAGE:
                un_p.extend([int(block_table[b, j])] * (PAGE - first))
                un_s.extend(range(first, PAGE))
    if has_poison:
        un_p.extend([poison] * PAGE)
        un_s.extend(range(PAGE))
    un_p = torch.tensor(un_p, dtype=torch.long, device=kc.device)
    un_s = torch.tensor(un_s, dtype=torch.long, device=kc.device)
    k_scale = v_scale = 1.0
    if kv_dtype == "bf16":
        nan = torch.tensor(BF16_NAN, dtype=torch.int16).view(torch.bfloat16).to(kc.device)
        kc[un_p, :, un_s, :] = nan
        vc[un_p, :, un_s, :] = nan
    elif kv_dtype == "fp8":
        if fp8_scales is None:
            k_scale = float(np.float32(max(_amax(kc), 1e-3) / 448.0))
            v_scale = float(np.float32(max(_amax(vc), 1e-3) / 448.0))
        else:
            k_scale, v_scale = (float(np.float32(x)) for x in fp8_scales)
        kc = _fp8_codes(kc, k_scale)
        vc = _fp8_codes(vc, v_scale)
        kc[un_p, :, un_s, :] = FP8_NAN
        vc[un_p, :, un_s, :] = FP8_NAN
    else:
        raise ValueError(kv_dtype)

    q_start = np.zeros(B + 1, dtype=np.int32)
    q_start[1:] = np.cumsum(q_lens)
    return LayerCall(name=name, kind=kind, kv_dtype=kv_dtype, q_start=q_start,
                     kv_len=kv_lens.astype(np.int32), block_table=block_table, q=q, k=k,
                     v=v, gate=gate, q_norm_w=q_norm_w, k_norm_w=k_norm_w,
                     gate_bias=gate_bias, k_cache=kc, v_cache=vc, k_scale=k_scale,
                     v_scale=v_scale, poison_page=poison)


def _normal_bf16(n: int, key) -> torch.Tensor:
    """n standard normals rounded to bf16 by torch's cast, drawn chunk by chunk like
    _normal_f32 (same values), without holding the float32 copy whole."""
    out = torch.empty(n, dtype=torch.bfloat16)
    nchunks = (n + _CHUNK - 1) // _CHUNK

    def fill(i):
        s, e = i * _CHUNK, min(n, (i + 1) * _CHUNK)
        a = np.random.default_rng(list(key) + [i]).standard_normal(e - s, dtype=np.float32)
        out[s:e] = torch.from_numpy(a).to(torch.bfloat16)

    with ThreadPoolExecutor(_THREADS) as ex:
        list(ex.map(fill, range(nchunks)))
    return out


def _normal_bf16_device(n: int, key, device) -> torch.Tensor:
    """n standard normals rounded to bf16, drawn on `device` by torch's Philox generator
    seeded from `key`, chunk by chunk."""
    out = torch.empty(n, dtype=torch.bfloat16, device=device)
    gen = torch.Generator(device=device)
    seed = 0
    for k in key:
        seed = (seed * 1000003 + int(k) + 1) % (1 << 62)
    gen.manual_seed(seed)
    step = 1 << 26
    for s in range(0, n, step):
        e = min(n, s + step)
        out[s:e] = torch.randn(e - s, generator=gen, device=device, dtype=torch.float32).to(torch.bfloat16)
    return out


def _amax(x: torch.Tensor) -> float:
    flat = x.reshape(-1)
    step = 1 << 26
    m = 0.0
    for s in range(0, flat.numel(), step):
        m = max(m, float(flat[s:s + step].float().abs().max()))
    return m


def _fp8_codes(x_bf16: torch.Tensor, scale: float) -> torch.Tensor:
    """fp8 e4m3 codes of cached values x/scale (torch's cast after an explicit clamp)."""
    out = torch.empty(x_bf16.shape, dtype=torch.uint8, device=x_bf16.device)
    flat_x = x_bf16.reshape(-1)
    flat_o = out.view(-1)
    step = 1 << 26
    for s in range(0, flat_x.numel(), step):
        xs = flat_x[s:s + step].float() / scale
        flat_o[s:s + step] = xs.clamp(-448.0, 448.0).to(torch.float8_e4m3fn).view(torch.uint8)
    return out


# ----------------------------------------------------------------------------------
# The five workloads
# ----------------------------------------------------------------------------------

def config_shapes(cfg: int):
    """(q_lens, kv_lens, kv_dtype, description) of workload `cfg`."""
    if cfg == 0:
        return [1024], [1024], "bf16", "tiny prefill: 1 x 1024 new tokens, no cache"
    if cfg == 1:
        return [2048] * 8, [98304 + 2048] * 8, "bf16", "long prefill: 8 x 2048 new on 98304 cached"
    if cfg == 2:
        return [1], [100000], "bf16", "batch-1 decode at p = 100000 (99999 cached + 1 new)"
    if cfg == 3:
        L = np.random.default_rng(3).integers(8192, 131072, 32, endpoint=True)
        return [1] * 32, list(L), "fp8", "batched decode: 32 seqs, L ~ U[8K,128K], fp8 KV"
    if cfg == 4:
        return [8], [1048576 + 8], "fp8", "1M-token verify: 8-token causal block on 1048576 cached, fp8 KV"
    raise ValueError(cfg)


def make_config(cfg: int, kind: str, seed: int | None = None, cache_device=None,
                heads=None, kv_dtype: str | None = None) -> LayerCall:
    """Workload `cfg` (0..4) for one layer kind ("swa" or "full"); seed defaults to cfg.
    heads = (Hq, Hkv) draws the same shapes with other head counts (see make_call);
    kv_dtype ("bf16" / "fp8") replaces the workload's cache dtype."""
    q_lens, kv_lens, cfg_dtype, desc = config_shapes(cfg)
    kv_dtype = cfg_dtype if kv_dtype is None else kv_dtype
    seed = cfg if seed is None else seed
    call = make_call(q_lens, kv_lens, kind, kv_dtype, [seed, 0 if kind == "swa" else 1],
                     name=f"config{cfg}-{kind}", cache_device=cache_device, heads=heads)
    call.extra["description"] = desc
    return call


def make_linear(m: int, n: int, k: int, seed, device=None):
    """Inputs of one projection y = x W^T: x [m, k] ~ N(0,1) and W [n, k] ~ N(0,1)/sqrt(k),
    both rounded to bf16 by torch's cast (so y has unit scale). With device set, both are
    drawn there by torch's seeded generator."""
    key = [int(s) for s in (seed if isinstance(seed, (list, tuple)) else [seed])]
    if device is None:
        x = _bf16(_normal_f32(m * k, key + [1])).view(m, k)
        w = _bf16(_normal_f32(n * k, key + [2]) / np.float32(math.sqrt(k))).view(n, k)
        return x, w
    g = torch.Generator(device=device)
    g.manual_seed(int(np.random.default_rng(key + [1]).integers(1 << 62)))
    x = torch.randn(m, k, generator=g, device=device, dtype=torch.float32).to(torch.bfloat16)
    w = (torch.randn(n, k, generator=g, device=device, dtype=torch.float32) / math.sqrt(k)).to(torch.bfloat16)
    return x, w
