"""Helpers shared by the GPU tests: stage a synthetic layer call on the device, run the
HIP path through the C ABI, and compare with the oracle."""

from __future__ import annotations

import sys

import numpy as np
import torch

import oracle.beam_oracle as O

# Output tolerances of the specification (max-abs, mean-abs), by cache dtype.
TOL = {"bf16": (2e-2, 2e-3), "fp8": (6e-2, 6e-3)}


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def bits16(t: torch.Tensor) -> np.ndarray:
    return t.detach().contiguous().cpu().view(torch.int16).numpy().view(np.uint16)


def ordered16(bits) -> np.ndarray:
    b = np.asarray(bits).astype(np.int64)
    return np.where(b & 0x8000, -(b & 0x7FFF), b)


def ordered8(codes) -> np.ndarray:
    b = np.asarray(codes).astype(np.int64)
    return np.where(b & 0x80, -(b & 0x7F), b)


def stage(call, device="cuda"):
    from nope_gqa_attention_amd import beamattn as ba
    from nope_gqa_attention_amd.layer import HybridAttention

    d = {"batch": ba.DeviceBatch(call.q_start, call.kv_len, call.block_table, device),
         "cache": ba.DeviceCache(call.k_cache.to(device), call.v_cache.to(device),
                                 call.k_scale, call.v_scale),
         "layer": HybridAttention(call.kind, num_q_heads=call.num_q_heads,
                                  num_kv_heads=call.num_kv_heads)}
    for name in ("q", "k", "v", "gate", "q_norm_w", "k_norm_w", "gate_bias"):
        d[name] = getattr(call, name).to(device)
    d["q_out"] = torch.empty_like(d["q"])
    d["out"] = torch.empty_like(d["q"])
    return d


def run_kvwrite(d):
    d["layer"].kvwrite(d["batch"], d["cache"], d["q"], d["k"], d["v"], d["q_norm_w"],
                       d["k_norm_w"], d["q_out"])


def run_attend(d, mode="auto", gate=True):
    d["layer"].attend(d["batch"], d["cache"], d["q_out"], d["gate"] if gate else None,
                      d["gate_bias"] if gate else None, d["out"], mode=mode)


def run_layer(call, mode="auto"):
    d = stage(call)
    run_kvwrite(d)
    run_attend(d, mode)
    torch.cuda.synchronize()
    return d


def assert_close_to_oracle(gpu_out_bits, y_ref, kv_dtype, what=""):
    g = O.bf16_bits_to_f64(gpu_out_bits)
    assert np.all(np.isfinite(g)), f"{what}: non-finite GPU output"
    err = np.abs(g - y_ref)
    mx, mean = float(err.max()), float(err.mean())
    tmax, tmean = TOL[kv_dtype]
    say(f"  {what}: max-abs {mx:.3e} (tol {tmax}), mean-abs {mean:.3e} (tol {tmean}), "
        f"rows {g.shape[0]}")
    assert mx <= tmax and mean <= tmean, f"{what}: max {mx} mean {mean}"
    return mx, mean


def seq_host_inputs(call, b: int):
    """Oracle inputs for sequence b of a (possibly device-resident, multi-GiB) call: only
    the pages its block table names are copied to the host, renumbered densely, so the
    oracle reads exactly the bytes the GPU read."""
    bt = np.asarray(call.block_table[b])
    pages, inv = np.unique(bt, return_inverse=True)
    idx = torch.from_numpy(pages.astype(np.int64)).to(call.k_cache.device)
    kc = call.k_cache[idx].cpu()
    vc = call.v_cache[idx].cpu()
    s, e = int(call.q_start[b]), int(call.q_start[b + 1])

    def bits(t):
        t = t.cpu()
        return t.view(torch.int16).numpy().view(np.uint16) if t.dtype == torch.bfloat16 else t.numpy()

    return {
        "kind": call.kind, "kv_dtype": call.kv_dtype,
        "q_start": np.array([0, e - s], dtype=np.int32), "kv_len": np.asarray(call.kv_len[b:b + 1]),
        "block_table": inv.astype(np.int32).reshape(1, -1),
        "q": bits(call.q[s:e]), "k": bits(call.k[s:e]), "v": bits(call.v[s:e]),
        "gate": bits(call.gate[s:e]), "q_norm_w": bits(call.q_norm_w),
        "k_norm_w": bits(call.k_norm_w), "gate_bias": bits(call.gate_bias),
        "k_cache": bits(kc), "v_cache": bits(vc),
        "k_scale": call.k_scale, "v_scale": call.v_scale,
    }
