"""One attention-layer call of the hybrid model through libbeamattn.

HybridAttention chains the C-ABI entry points the way a serving step uses them:
the fused Q/K norm + RoPE/SSMax + KV-store kernel, then prefill attention (any number
of new tokens) or split-K decode attention (1..16 new tokens per sequence), with the
sigmoid head gate fused into the attention epilogue. Buffers are torch tensors owned
by the caller; this class only marshals them.
"""

from __future__ import annotations

import torch

from . import beamattn as ba


class HybridAttention:
    def __init__(self, kind: str, num_q_heads: int = 48, num_kv_heads: int = 8, window: int = 512,
                 rope_theta: float = 1.0e4, rms_eps: float = 1.0e-6, ssmax_base: float = 2048.0,
                 ssmax_exponent: float = 0.1, sm_scale: float | None = None):
        self.kind = kind
        self.desc = ba.layer_desc(kind, num_q_heads, num_kv_heads, window, rope_theta, rms_eps,
                                  ssmax_base, ssmax_exponent, sm_scale)
        self._ws = None

    def workspace(self, batch: ba.DeviceBatch) -> torch.Tensor | None:
        need = ba.beam_attn_decode_workspace_bytes(self.desc, batch.num_seqs, batch.max_q_len,
                                                   batch.max_kv_len)
        if need == 0:
            return None
        if self._ws is None or self._ws.numel() < need:
            self._ws = torch.empty(need, dtype=torch.uint8, device=batch.kv_len.device)
        return self._ws

    def kvwrite(self, batch, cache, q, k, v, q_norm_w, k_norm_w, q_out, stream=None):
        ba.beam_qknorm_rope_ssmax_kvwrite(self.desc, batch, cache, q, k, v, q_norm_w, k_norm_w,
                                          q_out, stream=stream)

    def attend(self, batch, cache, q_prepared, gate, gate_bias, out, mode: str = "auto", stream=None):
        use_decode = mode == "decode" or (mode == "auto" and 1 <= batch.max_q_len <= 16)
        if use_decode:
            ba.beam_attn_decode(self.desc, batch, cache, q_prepared, gate, gate_bias, out,
                                self.workspace(batch), stream=stream)
        else:
            ba.beam_attn_prefill(self.desc, batch, cache, q_prepared, gate, gate_bias, out,
                                 stream=stream)

    def forward(self, batch, cache, q, k, v, q_norm_w, k_norm_w, gate, gate_bias, q_out=None,
                out=None, mode: str = "auto", stream=None):
        """kvwrite then attention; returns the gated output [N, Hq, 128] bf16."""
        q_out = torch.empty_like(q) if q_out is None else q_out
        out = torch.empty_like(q) if out is None else out
        self.kvwrite(batch, cache, q, k, v, q_norm_w, k_norm_w, q_out, stream=stream)
        self.attend(batch, cache, q_out, gate, gate_bias, out, mode=mode, stream=stream)
        return out
