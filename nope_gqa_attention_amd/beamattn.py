"""Thin Python binding of libbeamattn (include/beamattn.h), same names as the C ABI.

Argument marshalling only: torch tensors supply device pointers, element strides and
the current HIP stream; every step of the computation runs in the library's HIP
kernels. There is no fallback: if the library is missing or cannot be loaded, or the
process maps a second HIP runtime, load() raises.
"""

from __future__ import annotations

import ctypes
import math
import os
from ctypes import c_float, c_int32, c_int64, c_size_t, c_uint64, c_void_p

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libbeamattn.so")
# the same library built with BEAMATTN_DEBUG: the K/V-write, prefill and decode entry
# points also check the device-side batch metadata (synchronously) before launching
DEBUG_LIB_PATH = os.path.join(HERE, "libbeamattn_debug.so")

BEAM_ABI_VERSION = 2
BEAM_OK, BEAM_ERR_INVALID_ARG, BEAM_ERR_UNSUPPORTED, BEAM_ERR_WORKSPACE, BEAM_ERR_HIP = range(5)
BEAM_LAYER_SWA, BEAM_LAYER_FULL = 0, 1
BEAM_KV_BF16, BEAM_KV_FP8_E4M3 = 0, 1

ENTRY_POINTS = (
    "beam_qknorm_rope_ssmax_kvwrite", "beam_attn_prefill", "beam_attn_decode",
    "beam_attn_decode_noalloc", "beam_attn_decode_workspace_bytes", "beam_head_gate",
    "beam_linear_bf16",
    "beam_kv_bytes_per_token",
    "beam_status_string", "beam_last_error", "beam_abi_version",
)


class BeamError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{_STATUS_NAMES.get(status, status)}: {message}")
        self.status = status


_STATUS_NAMES = {1: "BEAM_ERR_INVALID_ARG", 2: "BEAM_ERR_UNSUPPORTED", 3: "BEAM_ERR_WORKSPACE",
                 4: "BEAM_ERR_HIP"}


class LayerDesc(ctypes.Structure):
    _fields_ = [("num_q_heads", c_int32), ("num_kv_heads", c_int32), ("head_dim", c_int32),
                ("page_size", c_int32), ("kind", c_int32), ("window", c_int32),
                ("rope_theta", c_float), ("rms_eps", c_float), ("ssmax_base", c_float),
                ("ssmax_exponent", c_float), ("sm_scale", c_float)]


class KVCache(ctypes.Structure):
    _fields_ = [("k", c_void_p), ("v", c_void_p), ("num_pages", c_int64), ("dtype", c_int32),
                ("k_scale", c_float), ("v_scale", c_float)]


class Batch(ctypes.Structure):
    _fields_ = [("num_seqs", c_int32), ("q_start", c_void_p), ("kv_len", c_void_p),
                ("block_table", c_void_p), ("max_pages", c_int32), ("max_q_len", c_int32),
                ("max_kv_len", c_int64), ("num_tokens", c_int64)]


_lib = None


def _hip_runtimes_mapped():
    paths = set()
    try:
        with open("/proc/self/maps") as f:
            for line in f:
                if "libamdhip64" in line:
                    paths.add(os.path.realpath(line.split()[-1]))
    except OSError:
        pass
    return paths


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libbeamattn once (after torch, so that both share torch's HIP runtime)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"libbeamattn not built: {path} is missing "
                           "(run `python -m nope_gqa_attention_amd.build`)")
    lib = ctypes.CDLL(path)
    P = ctypes.POINTER
    lib.beam_qknorm_rope_ssmax_kvwrite.argtypes = [
        P(LayerDesc), P(Batch), P(KVCache), c_void_p, c_int64, c_void_p, c_int64, c_void_p,
        c_int64, c_void_p, c_void_p, c_int64, c_void_p, c_int64, c_void_p]
    lib.beam_qknorm_rope_ssmax_kvwrite.restype = c_int32
    lib.beam_attn_prefill.argtypes = [
        P(LayerDesc), P(Batch), P(KVCache), c_void_p, c_int64, c_void_p, c_int64, c_void_p,
        c_void_p, c_int64, c_void_p]
    lib.beam_attn_prefill.restype = c_int32
    lib.beam_attn_decode.argtypes = [
        P(LayerDesc), P(Batch), P(KVCache), c_void_p, c_int64, c_void_p, c_int64, c_void_p,
        c_void_p, c_int64, c_void_p, c_size_t, c_void_p]
    lib.beam_attn_decode.restype = c_int32
    lib.beam_attn_decode_noalloc.argtypes = [
        P(LayerDesc), P(Batch), P(KVCache), c_void_p, c_int64, c_void_p, c_int64, c_void_p,
        c_void_p, c_int64, c_void_p]
    lib.beam_attn_decode_noalloc.restype = c_int32
    lib.beam_attn_decode_workspace_bytes.argtypes = [P(LayerDesc), c_int32, c_int32, c_int64]
    lib.beam_attn_decode_workspace_bytes.restype = c_size_t
    lib.beam_head_gate.argtypes = [
        P(LayerDesc), c_int64, c_void_p, c_int64, c_void_p, c_int64, c_void_p, c_void_p, c_int64,
        c_void_p]
    lib.beam_head_gate.restype = c_int32
    lib.beam_linear_bf16.argtypes = [c_int64, c_int64, c_int64, c_void_p, c_int64, c_void_p,
                                     c_int64, c_void_p, c_int64, c_void_p]
    lib.beam_linear_bf16.restype = c_int32
    lib.beam_kv_bytes_per_token.argtypes = [c_int32, c_int32, c_int32, c_int32]
    lib.beam_kv_bytes_per_token.restype = c_uint64
    lib.beam_status_string.argtypes = [c_int32]
    lib.beam_status_string.restype = ctypes.c_char_p
    lib.beam_last_error.argtypes = []
    lib.beam_last_error.restype = ctypes.c_char_p
    lib.beam_abi_version.argtypes = []
    lib.beam_abi_version.restype = c_int32
    if lib.beam_abi_version() != BEAM_ABI_VERSION:
        raise RuntimeError(f"libbeamattn ABI {lib.beam_abi_version()} != {BEAM_ABI_VERSION}")
    runtimes = _hip_runtimes_mapped()
    if len(runtimes) > 1:
        raise RuntimeError(f"two HIP runtimes mapped in this process: {sorted(runtimes)}; "
                           "import torch before loading libbeamattn")
    _lib = lib
    return lib


# ------------------------------------------------------------------ descriptors

def layer_desc(kind: str, num_q_heads: int = 48, num_kv_heads: int = 8, window: int = 512,
               rope_theta: float = 1.0e4, rms_eps: float = 1.0e-6, ssmax_base: float = 2048.0,
               ssmax_exponent: float = 0.1, sm_scale: float | None = None) -> LayerDesc:
    k = {"swa": BEAM_LAYER_SWA, "full": BEAM_LAYER_FULL}[kind]
    return LayerDesc(num_q_heads, num_kv_heads, 128, 64, k, window if k == BEAM_LAYER_SWA else 0,
                     rope_theta, rms_eps, ssmax_base, ssmax_exponent,
                     1.0 / math.sqrt(128.0) if sm_scale is None else sm_scale)


class DeviceBatch:
    """Device copies of a batch's index arrays plus the host bounds the ABI needs."""

    def __init__(self, q_start, kv_len, block_table, device="cuda"):
        qs = torch.as_tensor(q_start, dtype=torch.int32)
        kl = torch.as_tensor(kv_len, dtype=torch.int32)
        bt = torch.as_tensor(block_table, dtype=torch.int32)
        self.q_start = qs.to(device).contiguous()
        self.kv_len = kl.to(device).contiguous()
        self.block_table = bt.to(device).contiguous()
        q_lens = (qs[1:] - qs[:-1]) if len(kl) else torch.zeros(0, dtype=torch.int32)
        self.num_seqs = len(kl)
        self.num_tokens = int(qs[-1]) if len(qs) else 0
        self.max_q_len = int(q_lens.max()) if len(kl) else 0
        self.max_kv_len = int(kl.max()) if len(kl) else 0
        self.max_pages = int(bt.shape[1]) if bt.dim() == 2 else 0

    def struct(self) -> Batch:
        return Batch(self.num_seqs, self.q_start.data_ptr(), self.kv_len.data_ptr(),
                     self.block_table.data_ptr(), self.max_pages, self.max_q_len,
                     self.max_kv_len, self.num_tokens)


class DeviceCache:
    """One layer's paged K/V cache: [num_pages, Hkv, 64, 128] bf16, or uint8 fp8 codes."""

    def __init__(self, k: torch.Tensor, v: torch.Tensor, k_scale: float = 1.0, v_scale: float = 1.0):
        assert k.shape == v.shape and k.dtype == v.dtype and k.is_contiguous() and v.is_contiguous()
        self.k, self.v = k, v
        self.dtype = BEAM_KV_BF16 if k.dtype == torch.bfloat16 else BEAM_KV_FP8_E4M3
        if self.dtype == BEAM_KV_FP8_E4M3:
            assert k.dtype == torch.uint8
        self.k_scale, self.v_scale = float(k_scale), float(v_scale)

    def struct(self) -> KVCache:
        return KVCache(self.k.data_ptr(), self.v.data_ptr(), self.k.shape[0], self.dtype,
                       self.k_scale, self.v_scale)


# ------------------------------------------------------------------ marshalling helpers

def _stream(stream):
    if stream is None:
        return c_void_p(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, torch.cuda.Stream):
        return c_void_p(stream.cuda_stream)
    return c_void_p(int(stream))


def _tok(t: torch.Tensor | None, name: str):
    """(pointer, token stride in elements) of a [N, H, 128] or [N, H*128] tensor whose
    head values are contiguous within each token."""
    if t is None:
        return None, 0
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if t.dim() == 3:
        if t.stride(2) != 1 or t.stride(1) != t.shape[2]:
            raise ValueError(f"{name}: heads must be contiguous within a token")
    elif t.dim() == 2:
        if t.stride(1) != 1:
            raise ValueError(f"{name}: values must be contiguous within a token")
    elif t.dim() != 1:
        raise ValueError(f"{name}: expected [N, H, D], [N, H*D] or [D]")
    return c_void_p(t.data_ptr()), (t.stride(0) if t.dim() > 1 else 0)


def _check(status: int):
    if status != BEAM_OK:
        raise BeamError(status, load().beam_last_error().decode())


# ------------------------------------------------------------------ entry points

def beam_qknorm_rope_ssmax_kvwrite(layer: LayerDesc, batch: DeviceBatch, cache: DeviceCache,
                                   q, k, v, q_norm_w, k_norm_w, q_out, norm_w_head_stride: int = 0,
                                   stream=None):
    lib = load()
    qp, qs = _tok(q, "q")
    kp, ks = _tok(k, "k")
    vp, vs = _tok(v, "v")
    op, os_ = _tok(q_out, "q_out")
    b, c = batch.struct(), cache.struct()
    _check(lib.beam_qknorm_rope_ssmax_kvwrite(
        ctypes.byref(layer), ctypes.byref(b), ctypes.byref(c), qp, qs, kp, ks, vp, vs,
        c_void_p(q_norm_w.data_ptr()), c_void_p(k_norm_w.data_ptr()), norm_w_head_stride, op, os_,
        _stream(stream)))


def beam_attn_prefill(layer: LayerDesc, batch: DeviceBatch, cache: DeviceCache, q, gate,
                      gate_bias, out, stream=None):
    lib = load()
    qp, qs = _tok(q, "q")
    gp, gs = _tok(gate, "gate")
    op, os_ = _tok(out, "out")
    b, c = batch.struct(), cache.struct()
    _check(lib.beam_attn_prefill(
        ctypes.byref(layer), ctypes.byref(b), ctypes.byref(c), qp, qs, gp, gs,
        c_void_p(gate_bias.data_ptr() if gate_bias is not None else None), op, os_, _stream(stream)))


def beam_attn_decode_workspace_bytes(layer: LayerDesc, num_seqs: int, max_q_len: int,
                                     max_kv_len: int) -> int:
    return int(load().beam_attn_decode_workspace_bytes(ctypes.byref(layer), num_seqs, max_q_len,
                                                       max_kv_len))


def beam_attn_decode(layer: LayerDesc, batch: DeviceBatch, cache: DeviceCache, q, gate,
                     gate_bias, out, workspace: torch.Tensor | None, stream=None):
    lib = load()
    qp, qs = _tok(q, "q")
    gp, gs = _tok(gate, "gate")
    op, os_ = _tok(out, "out")
    b, c = batch.struct(), cache.struct()
    wp = c_void_p(workspace.data_ptr()) if workspace is not None else c_void_p(None)
    wb = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(lib.beam_attn_decode(
        ctypes.byref(layer), ctypes.byref(b), ctypes.byref(c), qp, qs, gp, gs,
        c_void_p(gate_bias.data_ptr() if gate_bias is not None else None), op, os_, wp, wb,
        _stream(stream)))


BEAM_DECODE_NOALLOC_SCRATCH_BYTES = 32 * 1024 * 1024


def beam_attn_decode_noalloc(layer: LayerDesc, batch: DeviceBatch, cache: DeviceCache, q, gate,
                             gate_bias, out, stream=None):
    """beam_attn_decode with the split partials in the library's per-device scratch array
    (no workspace argument, no allocation)."""
    lib = load()
    qp, qs = _tok(q, "q")
    gp, gs = _tok(gate, "gate")
    op, os_ = _tok(out, "out")
    b, c = batch.struct(), cache.struct()
    _check(lib.beam_attn_decode_noalloc(
        ctypes.byref(layer), ctypes.byref(b), ctypes.byref(c), qp, qs, gp, gs,
        c_void_p(gate_bias.data_ptr() if gate_bias is not None else None), op, os_,
        _stream(stream)))


def beam_head_gate(layer: LayerDesc, attn, gate, gate_bias, out, stream=None):
    lib = load()
    ap, as_ = _tok(attn, "attn")
    gp, gs = _tok(gate, "gate")
    op, os_ = _tok(out, "out")
    n = attn.shape[0]
    _check(lib.beam_head_gate(ctypes.byref(layer), n, ap, as_, gp, gs,
                              c_void_p(gate_bias.data_ptr()), op, os_, _stream(stream)))


def beam_linear_bf16(x, w, y, stream=None):
    """y = x w^T: x [m, k], w [n, k], y [m, n] bf16 CUDA tensors with unit column stride
    (row strides free, e.g. column ranges of a wider tensor)."""
    for name, t in (("x", x), ("w", w), ("y", y)):
        if t.dtype != torch.bfloat16 or t.dim() != 2 or t.stride(1) != 1 or not t.is_cuda:
            raise ValueError(f"{name} must be a 2-D bf16 CUDA tensor with unit column stride")
    m, k = x.shape
    n = w.shape[0]
    if w.shape[1] != k or tuple(y.shape) != (m, n):
        raise ValueError(f"shape mismatch: x {tuple(x.shape)}, w {tuple(w.shape)}, y {tuple(y.shape)}")
    _check(load().beam_linear_bf16(m, n, k, c_void_p(x.data_ptr()), x.stride(0),
                                   c_void_p(w.data_ptr()), w.stride(0), c_void_p(y.data_ptr()),
                                   y.stride(0), _stream(stream)))


def beam_kv_bytes_per_token(num_full_layers: int, num_kv_heads: int, head_dim: int, dtype: int) -> int:
    return int(load().beam_kv_bytes_per_token(num_full_layers, num_kv_heads, head_dim, dtype))


def beam_status_string(status: int) -> str:
    return load().beam_status_string(status).decode()


def beam_last_error() -> str:
    return load().beam_last_error().decode()


def beam_abi_version() -> int:
    return int(load().beam_abi_version())


def workspace_for(layer: LayerDesc, batch: DeviceBatch, device="cuda") -> torch.Tensor | None:
    """A caller-owned decode workspace of the required size (256-byte aligned by torch)."""
    nbytes = beam_attn_decode_workspace_bytes(layer, batch.num_seqs, batch.max_q_len, batch.max_kv_len)
    if nbytes == 0:
        return None
    return torch.empty(nbytes, dtype=torch.uint8, device=device)
