"""Benchmark of the hybrid SWA / NoPE attention core on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-decode] [--no-cpu-baseline]

One step = one pass of the attention hot path over the long-prefill workload: 8
sequences, each adding 2,048 new tokens on top of 98,304 cached tokens (64-token
pages in shuffled physical order, bf16 KV), through both layer kinds:
  full NoPE/SSMax layer: fused Q/K norm + SSMax + KV store, then prefill attention
                         with the fused sigmoid head gate;
  sliding-window layer:  fused Q/K norm + RoPE + KV store, then prefill attention
                         (window 512) with the gate.
All inputs are seeded synthetic tensors already resident in HBM when the timed region
starts. The printed JSON line reports new tokens per second through the step, the
roofline of the dominant kernel (full-layer prefill, bf16 MFMA) measured with HIP
events on its stream, per-layer figures, the decode / verify workloads (HBM roofline),
and the fp64 CPU oracle timed on a bounded sample of the same workload.
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HQ, HKV, D = 48, 8, 128
PEAK_BF16_TFLOPS = 2500.0        # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0            # MI355X HBM3E
PREFILL_SRC = os.path.join(ROOT, "nope_gqa_attention_amd", "csrc", "attn_prefill.hip")
TRAFFIC_SUMMARY = os.path.join(ROOT, "profiles", "prefill_full_8x2048_on_98304_hbm_traffic.md")
CALIBRATION_BYTES = 1 << 30      # the plain device-to-device copy run by --copy-calibration


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def file_sha256(path):
    import hashlib

    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def summarize_counters(paths):
    """Markdown summary of rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE counter CSVs of a bench
    run with --copy-calibration: per libbeamattn kernel and launch size, the mean KiB per
    dispatch of each counter, the HBM bytes they stand for once scaled by what the same
    counter read for the plain 1 GiB copy, and the rate those bytes give over the
    dispatch's own duration. Ends with the record the bench line's roofline.traffic is read
    from, tagged with the hash of the prefill kernel source it was measured on."""
    import collections
    import csv
    import re

    per = collections.defaultdict(lambda: collections.defaultdict(list))
    calib = {}
    for path in paths:
        for r in csv.DictReader(open(path)):
            name, ctr, val = r["Kernel_Name"], r["Counter_Name"], float(r["Counter_Value"])
            if "copyBuffer" in name:
                calib[ctr] = max(calib.get(ctr, 0.0), val)
            elif "beam::" in name:
                short = re.sub(r"\(.*", "", name.replace("(anonymous namespace)::", ""))
                short = short.replace("void ", "")
                key = (short, int(r["Grid_Size"]) // int(r["Workgroup_Size"]))
                per[key][ctr].append(val)
                per[key]["dur_" + ctr].append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-9)
    factor = {c: CALIBRATION_BYTES / 1024 / v for c, v in calib.items() if v > 0}
    lines = ["| kernel | workgroups | dispatches | FETCH_SIZE KiB | WRITE_SIZE KiB | HBM GB per dispatch | "
             "HBM GB/s over the dispatch |", "|---|---|---|---|---|---|---|"]
    record = None
    mean = lambda v: sum(v) / len(v) if v else None
    for (k, wgs) in sorted(per):
        c = per[(k, wgs)]
        fm, wm = mean(c.get("FETCH_SIZE", [])), mean(c.get("WRITE_SIZE", []))
        gb = gbs = None
        if fm is not None and wm is not None and factor.get("FETCH_SIZE") and factor.get("WRITE_SIZE"):
            fb, wb = fm * factor["FETCH_SIZE"] * 1024, wm * factor["WRITE_SIZE"] * 1024
            gb = (fb + wb) / 1e9
            gbs = fb / mean(c["dur_FETCH_SIZE"]) / 1e9 + wb / mean(c["dur_WRITE_SIZE"]) / 1e9
        n = max(len(c.get("FETCH_SIZE", [])), len(c.get("WRITE_SIZE", [])))
        lines.append(f"| {k} | {wgs} | {n} | {fm if fm is None else round(fm, 1)} | "
                     f"{wm if wm is None else round(wm, 1)} | {gb if gb is None else round(gb, 3)} | "
                     f"{gbs if gbs is None else round(gbs, 1)} |")
        # the full NoPE layer over a bf16 cache: prefill_kernel<BEAM_LAYER_FULL, BEAM_KV_BF16>
        if re.search(r"prefill_kernel<1(, 0)?>$", k) and gb is not None and record is None:
            record = round(gb * 1e9)
    lines.append("")
    lines.append(f"calibration (1 GiB copy): FETCH_SIZE {calib.get('FETCH_SIZE')} KiB -> factor "
                 f"{round(factor.get('FETCH_SIZE', 0), 4)}; WRITE_SIZE {calib.get('WRITE_SIZE')} KiB "
                 f"-> factor {round(factor.get('WRITE_SIZE', 0), 4)}")
    if record is not None:
        lines.append(f"traffic-record: kernel=prefill_kernel<1,0> bytes_per_launch={record} "
                     f"source_sha256={file_sha256(PREFILL_SRC)}")
    return "\n".join(lines)


def summarize_trace(path):
    """Markdown table of a rocprofv3 --kernel-trace CSV (`*_kernel_trace.csv`): per
    libbeamattn kernel and launch shape (workgroups in x, y, z; threads per workgroup),
    the number of dispatches and their mean / min / max duration in microseconds."""
    import collections
    import csv
    import re

    groups = collections.defaultdict(list)
    for r in csv.DictReader(open(path)):
        name = r["Kernel_Name"]
        if "beam::" not in name:
            continue
        short = re.sub(r"\(.*", "", name.replace("(anonymous namespace)::", "").replace("void ", ""))
        wg = int(r["Workgroup_Size_X"])
        grid = (int(r["Grid_Size_X"]) // wg, int(r["Grid_Size_Y"]), int(r["Grid_Size_Z"]))
        groups[(short, grid, wg)].append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    lines = ["| kernel | workgroups (x, y, z) | threads | calls | average us | min us | max us |",
             "|---|---|---|---|---|---|---|"]
    for (k, grid, wg), d in sorted(groups.items(), key=lambda kv: -sum(kv[1])):
        lines.append(f"| {k} | {grid} | {wg} | {len(d)} | {sum(d) / len(d):.2f} | {min(d):.2f} | "
                     f"{max(d):.2f} |")
    return "\n".join(lines)


def summarize_mfma(paths):
    """Markdown summary of rocprofv3 --pmc runs with the derived counters MfmaUtil and
    MfmaFlopsBF16 and the raw GRBM_GUI_ACTIVE (one pass each): per libbeamattn kernel and
    launch size, the bf16 MFMA FLOPs the hardware counted per dispatch, the rate they give
    over the dispatch's duration (against the 2.5 PFLOP/s bf16 peak), the MFMA-busy share of
    SIMD cycles, and the engine clock (GRBM_GUI_ACTIVE is summed over the 8 XCDs)."""
    import collections
    import csv
    import re

    per = collections.defaultdict(lambda: collections.defaultdict(list))
    for path in paths:
        for r in csv.DictReader(open(path)):
            name = r["Kernel_Name"]
            if "beam::" not in name:
                continue
            short = re.sub(r"\(.*", "", name.replace("(anonymous namespace)::", "").replace("void ", ""))
            key = (short, int(r["Grid_Size"]) // int(r["Workgroup_Size"]))
            per[key][r["Counter_Name"]].append(float(r["Counter_Value"]))
            per[key]["dur_" + r["Counter_Name"]].append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-9)
    mean = lambda v: sum(v) / len(v) if v else None
    lines = ["| kernel | workgroups | dispatches | MFMA FLOP per dispatch (counted) | counted TFLOP/s | "
             "share of 2.5 PFLOP/s | MfmaUtil % | clock GHz |", "|---|---|---|---|---|---|---|---|"]
    for (k, wgs), c in sorted(per.items(), key=lambda kv: -(mean(kv[1].get("MfmaFlopsBF16", [])) or 0)):
        fl, util, gui = mean(c.get("MfmaFlopsBF16", [])), mean(c.get("MfmaUtil", [])), mean(c.get("GRBM_GUI_ACTIVE", []))
        tf = fl / mean(c["dur_MfmaFlopsBF16"]) / 1e12 if fl else None
        clk = gui / 8 / mean(c["dur_GRBM_GUI_ACTIVE"]) / 1e9 if gui else None
        n = max(len(v) for name, v in c.items() if not name.startswith("dur_"))
        fmt = lambda v, d: "" if v is None else f"{v:.{d}f}"
        lines.append(f"| {k} | {wgs} | {n} | {fmt(fl, 0)} | {fmt(tf, 1)} | "
                     f"{fmt(tf / PEAK_BF16_TFLOPS if tf else None, 4)} | {fmt(util, 1)} | {fmt(clk, 3)} |")
    return "\n".join(lines)


def recorded_traffic():
    """HBM bytes per launch of the full-layer prefill kernel from the committed counter
    summary, or None when that summary is missing or was taken on another version of the
    kernel source."""
    try:
        text = open(TRAFFIC_SUMMARY).read()
    except OSError:
        return None
    for line in text.splitlines():
        if line.startswith("traffic-record:"):
            kv = dict(tok.split("=", 1) for tok in line.split()[1:] if "=" in tok)
            if kv.get("source_sha256") == file_sha256(PREFILL_SRC):
                return int(kv["bytes_per_launch"])
    return None


def visible_pairs(q_lens, kv_lens, kind, window=512):
    """Visible (query token, key) pairs per head, summed over sequences."""
    total = 0
    for n, L in zip(q_lens, kv_lens):
        for i in range(int(n)):
            pos = int(L) - int(n) + i
            total += min(pos + 1, window) if kind == "swa" else pos + 1
    return total


def visible_keys_decode(q_lens, kv_lens, kind, window=512):
    """Distinct keys a decode call must read per sequence (union over its new tokens)."""
    total = 0
    for n, L in zip(q_lens, kv_lens):
        first = int(L) - int(n)
        lo = max(0, first - window + 1) if kind == "swa" else 0
        total += int(L) - lo
    return total


class Staged:
    """One layer call staged on the GPU."""

    def __init__(self, call, device="cuda"):
        import torch
        from nope_gqa_attention_amd import beamattn as ba
        from nope_gqa_attention_amd.layer import HybridAttention

        self.call = call
        self.batch = ba.DeviceBatch(call.q_start, call.kv_len, call.block_table, device)
        self.cache = ba.DeviceCache(call.k_cache.to(device), call.v_cache.to(device),
                                    call.k_scale, call.v_scale)
        self.layer = HybridAttention(call.kind, num_q_heads=call.num_q_heads,
                                     num_kv_heads=call.num_kv_heads)
        for n in ("q", "k", "v", "gate", "q_norm_w", "k_norm_w", "gate_bias"):
            setattr(self, n, getattr(call, n).to(device))
        self.q_out = torch.empty_like(self.q)
        self.out = torch.empty_like(self.q)
        self.ws = self.layer.workspace(self.batch) if call.max_q_len <= 16 else None

    def kvwrite(self):
        self.layer.kvwrite(self.batch, self.cache, self.q, self.k, self.v, self.q_norm_w,
                           self.k_norm_w, self.q_out)

    def attend(self, mode):
        self.layer.attend(self.batch, self.cache, self.q_out, self.gate, self.gate_bias, self.out,
                          mode=mode)


def timed_steps(parts, steps, warmup):
    """parts: list of (name, fn). Runs warmup + steps passes; returns (total ms per step,
    {name: mean ms per launch}) from HIP events recorded on torch's current stream, which
    is the stream every entry point is launched on."""
    import torch

    for _ in range(warmup):
        for _, fn in parts:
            fn()
    torch.cuda.synchronize()
    ev = {name: [] for name, _ in parts}
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(steps):
        for name, fn in parts:
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record()
            fn()
            b.record()
            ev[name].append((a, b))
    end.record()
    torch.cuda.synchronize()
    total = start.elapsed_time(end) / steps
    per = {name: sum(a.elapsed_time(b) for a, b in lst) / len(lst) for name, lst in ev.items()}
    return total, per


def oracle_threads():
    """Threads the oracle's BLAS pool uses (the rest of the oracle is single-threaded numpy)."""
    try:
        from threadpoolctl import threadpool_info
        return max((p.get("num_threads") or 0) for p in threadpool_info()) or os.cpu_count()
    except Exception:
        return os.cpu_count()


def host_inputs(call, seqs, kv_head=None):
    """Oracle inputs for sequences `seqs` of a staged call (possibly with multi-GiB caches
    on the device): only the pages their block tables name are copied to the host and
    renumbered densely, so the oracle reads exactly the bytes the GPU read. With kv_head
    set, only that KV head's cache and its query heads, gate columns and gate biases are
    kept (an exact 1/Hkv share of the attention work: heads are independent)."""
    import numpy as np
    import torch

    seqs = list(seqs)
    bt = np.asarray(call.block_table)[seqs]
    pages, inv = np.unique(bt, return_inverse=True)
    idx = torch.from_numpy(pages.astype(np.int64)).to(call.k_cache.device)
    hkv, hq = call.num_kv_heads, call.num_q_heads
    G = hq // hkv
    hs = slice(0, hkv) if kv_head is None else slice(kv_head, kv_head + 1)
    qh = slice(0, hq) if kv_head is None else slice(kv_head * G, (kv_head + 1) * G)
    kc = call.k_cache[idx][:, hs].contiguous().cpu()
    vc = call.v_cache[idx][:, hs].contiguous().cpu()
    qs = np.asarray(call.q_start)
    tok = np.concatenate([np.arange(qs[b], qs[b + 1]) for b in seqs]).astype(np.int64)
    n = [int(qs[b + 1] - qs[b]) for b in seqs]
    q_start = np.zeros(len(seqs) + 1, dtype=np.int32)
    q_start[1:] = np.cumsum(n)
    t = torch.from_numpy(tok)

    def bits(x):
        x = x.contiguous().cpu()
        return x.view(torch.int16).numpy().view(np.uint16) if x.dtype == torch.bfloat16 else x.numpy()

    gate = call.gate[t].view(len(tok), hq, D)[:, qh].reshape(len(tok), -1)
    return {
        "kind": call.kind, "kv_dtype": call.kv_dtype, "q_start": q_start,
        "kv_len": np.asarray(call.kv_len)[seqs], "block_table": inv.astype(np.int32).reshape(bt.shape),
        "q": bits(call.q[t][:, qh]), "k": bits(call.k[t][:, hs]), "v": bits(call.v[t][:, hs]),
        "gate": bits(gate), "q_norm_w": bits(call.q_norm_w), "k_norm_w": bits(call.k_norm_w),
        "gate_bias": bits(call.gate_bias[qh]), "k_cache": bits(kc), "v_cache": bits(vc),
        "k_scale": call.k_scale, "v_scale": call.v_scale,
    }


def time_oracle(inp, rows=None):
    """Seconds the fp64 oracle takes for one layer call (fused prepare + K/V store of every
    new token of `inp`, attention and gate for `rows`, all rows if None)."""
    import oracle.beam_oracle as O

    t0 = time.perf_counter()
    O.layer_call(inp, rows=rows)
    return time.perf_counter() - t0


def sample_rows(q_len, kv_len, count, seed):
    """Rows of one sequence's new tokens for a bounded oracle sample: the first and last
    token, the tokens that open a page, then seeded random ones, `count` in all."""
    import numpy as np

    first = kv_len - q_len
    rows = {0, q_len - 1} | {i for i in range(q_len) if (first + i) % 64 == 0}
    rest = [i for i in range(q_len) if i not in rows]
    rng = np.random.default_rng(seed)
    need = max(0, count - len(rows))
    rows |= set(int(x) for x in rng.choice(rest, size=min(need, len(rest)), replace=False))
    return np.array(sorted(rows)[:max(count, 2)], dtype=np.int64)


def oracle_long_prefill(staged, rows_per_seq):
    """The oracle on the long-prefill workload, per layer kind: every sequence, KV head 0
    and its 6 query heads, `rows_per_seq` sampled rows per sequence (all of its new tokens
    are still normed and stored). Extrapolated to all rows and heads by the visible
    (row, head, key) triples the sample covered, and labelled as extrapolated."""
    out = {}
    for kind, s in staged.items():
        call = s.call
        ql = [int(x) for x in call.q_lens]
        kl = [int(x) for x in call.kv_len]
        secs, pairs = 0.0, 0
        for b in range(call.num_seqs):
            inp = host_inputs(call, [b], kv_head=0)
            rows = sample_rows(ql[b], kl[b], rows_per_seq, 1000 + b)
            secs += time_oracle(inp, rows)
            pairs += sum(min(kl[b] - ql[b] + int(i) + 1, 512) if kind == "swa" else kl[b] - ql[b] + int(i) + 1
                         for i in rows)
        frac_heads = 1.0 / call.num_kv_heads
        total_pairs = visible_pairs(ql, kl, kind)
        scale = (total_pairs / pairs) / frac_heads
        out[kind] = {"sample_rows": rows_per_seq * call.num_seqs, "kv_heads_sampled": 1,
                     "sample_s": round(secs, 2), "extrapolated_full_s": round(secs * scale, 1),
                     "extrapolated_tokens_per_s": round(sum(ql) / (secs * scale), 3)}
        log(f"  oracle long prefill {kind}: {out[kind]}")
    return out


def run_decode(args, result, oracle_out=None):
    """The decode / verify workloads: batch-1 decode at p = 100,000 (bf16), 32 sequences
    of 8K..128K keys (fp8), and an 8-token verify block on 1,048,576 keys (fp8); each as
    a full NoPE layer and an SWA-512 layer (fused norm + KV store, then split-K decode
    attention with the gate)."""
    import torch

    import synth
    from nope_gqa_attention_amd import beamattn as ba

    dec = {}
    for cfg in (2, 3, 4):
        for kind in ("full", "swa"):
            call = synth.make_config(cfg, kind, cache_device="cuda")
            s = Staged(call)
            ql = [int(x) for x in call.q_lens]
            kl = [int(x) for x in call.kv_len]
            copies = [s]
            if cfg == 2 and kind == "full":
                # 409.6 MB of K/V would partly stay in the 256 MB MALL between
                # iterations: alternate between two copies at different addresses
                s2 = Staged(call)
                s2.cache = ba.DeviceCache(s.cache.k.clone(), s.cache.v.clone(),
                                          call.k_scale, call.v_scale)
                copies.append(s2)
            it = {"i": 0}

            def run_attn(copies=copies, it=it):
                c = copies[it["i"] % len(copies)]
                it["i"] += 1
                c.attend("decode")
            total, per_d = timed_steps([("kvwrite", s.kvwrite), ("decode", run_attn)],
                                       max(args.steps, 5) * 2, args.warmup)
            # the same step (kvwrite + decode) recorded once per cache copy as a HIP graph
            # and replayed: what a serving loop pays without per-launch host overhead
            graphs = []
            for c in copies:
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g):
                    c.kvwrite()
                    c.attend("decode")
                graphs.append(g)
            git = {"i": 0}

            def run_graph(graphs=graphs, git=git):
                graphs[git["i"] % len(graphs)].replay()
                git["i"] += 1
            _, per_g = timed_steps([("step", run_graph)], max(args.steps, 5) * 2, args.warmup)
            del graphs
            # attention alone, 20 calls back to back in one graph (cache copies alternating):
            # the device time per call without host launch overhead, which dominates the
            # eager timing of the latency-bound sliding-window calls
            n_rep = 20
            g20 = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g20):
                for r in range(n_rep):
                    copies[r % len(copies)].attend("decode")
            _, per_g20 = timed_steps([("rep", g20.replay)], max(args.steps, 5), args.warmup)
            del g20
            dev_ms = per_g20["rep"] / n_rep
            bpk = 2 * HKV * D * (2 if call.kv_dtype == "bf16" else 1)
            nbytes = visible_keys_decode(ql, kl, kind) * bpk
            gbs = nbytes / (per_d["decode"] * 1e-3) / 1e9
            dec[f"config{cfg}-{kind}"] = {
                "kv_dtype": call.kv_dtype, "seqs": len(ql), "q_len": max(ql),
                "decode_us": round(per_d["decode"] * 1e3, 2),
                "kvwrite_us": round(per_d["kvwrite"] * 1e3, 2),
                "kv_bytes": nbytes, "hbm_gbs": round(gbs, 1),
                "hbm_frac": round(gbs / PEAK_HBM_GBS, 4),
                "tokens_per_s": round(sum(ql) / ((per_d["decode"] + per_d["kvwrite"]) * 1e-3), 1),
                "step_eager_us": round((per_d["decode"] + per_d["kvwrite"]) * 1e3, 2),
                "step_graph_us": round(per_g["step"] * 1e3, 2),
                "decode_graph_us": round(dev_ms * 1e3, 2),
                "hbm_frac_graph": round(nbytes / (dev_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
            }
            log(f"  decode config{cfg}-{kind}: {dec[f'config{cfg}-{kind}']}")
            if oracle_out is not None:
                # the oracle on the same bytes, in full
                inp = host_inputs(call, range(call.num_seqs))
                full_s = time_oracle(inp)
                oracle_out[f"config{cfg}-{kind}"] = {
                    "s": round(full_s, 3), "tokens_per_s": round(sum(ql) / full_s, 3),
                    "sample": "in full",
                    "gpu_speedup": round(full_s / ((per_d["decode"] + per_d["kvwrite"]) * 1e-3), 1)}
                log(f"  oracle config{cfg}-{kind}: {oracle_out[f'config{cfg}-{kind}']}")
                del inp
            del s, copies, call
            torch.cuda.empty_cache()
    result["decode"] = dec



def run_tiny_prefill(args, result, oracle_out=None):
    """The tiny prefill workload (1 sequence, 1,024 new tokens, no cache) through both
    layer kinds: launch-bound at this size, reported beside the long prefill. Timed eagerly
    and as 20 back-to-back calls in one HIP graph (device time per call)."""
    import torch

    import synth

    res = {}
    for kind in ("full", "swa"):
        call = synth.make_config(0, kind)
        s = Staged(call)
        ql = [int(x) for x in call.q_lens]
        kl = [int(x) for x in call.kv_len]
        _, per = timed_steps([("kvwrite", s.kvwrite), ("attn", lambda s=s: s.attend("prefill"))],
                             max(args.steps, 10), args.warmup)
        n_rep = 20
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _ in range(n_rep):
                s.attend("prefill")
        _, pg = timed_steps([("rep", g.replay)], max(args.steps, 5), args.warmup)
        del g
        dev_ms = pg["rep"] / n_rep
        fl = 4 * D * HQ * visible_pairs(ql, kl, kind)
        res[kind] = {"prefill_us": round(per["attn"] * 1e3, 2), "kvwrite_us": round(per["kvwrite"] * 1e3, 2),
                     "prefill_graph_us": round(dev_ms * 1e3, 2), "algorithmic_gflop": round(fl / 1e9, 3),
                     "prefill_tflops_graph": round(fl / (dev_ms * 1e-3) / 1e12, 1),
                     "prefill_mfma_frac_graph": round(fl / (dev_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
                     "tokens_per_s": round(sum(ql) / ((per["attn"] + per["kvwrite"]) * 1e-3), 1)}
        log(f"  tiny prefill {kind}: {res[kind]}")
        if oracle_out is not None:
            secs = time_oracle(host_inputs(call, [0]))
            oracle_out[f"config0-{kind}"] = {
                "s": round(secs, 3), "tokens_per_s": round(sum(ql) / secs, 3), "sample": "in full",
                "gpu_speedup": round(secs / ((per["attn"] + per["kvwrite"]) * 1e-3), 1)}
            log(f"  oracle config0-{kind}: {oracle_out[f'config0-{kind}']}")
        del s, call
        torch.cuda.empty_cache()
    result["tiny_prefill"] = res


def run_prefill_fp8(args, result):
    """Chunked prefill over an fp8 KV cache: the long-prefill shapes (8 x 2048 new tokens
    on 98,304 cached) with the cache in fp8 e4m3, both layer kinds (fused store, then
    prefill attention with the codes widened to bf16 on their way into LDS)."""
    import torch

    import synth

    res = {}
    for kind in ("full", "swa"):
        call = synth.make_config(1, kind, cache_device="cuda", kv_dtype="fp8")
        s = Staged(call)
        ql = [int(x) for x in call.q_lens]
        kl = [int(x) for x in call.kv_len]
        _, per = timed_steps([("kvwrite", s.kvwrite), ("attn", lambda s=s: s.attend("prefill"))],
                             args.steps, args.warmup)
        tf = 4 * D * HQ * visible_pairs(ql, kl, kind) / (per["attn"] * 1e-3) / 1e12
        res[kind] = {"prefill_ms": round(per["attn"], 4), "kvwrite_ms": round(per["kvwrite"], 4),
                     "prefill_tflops": round(tf, 1), "prefill_mfma_frac": round(tf / PEAK_BF16_TFLOPS, 4)}
        log(f"  fp8-cache prefill {kind}: {res[kind]}")
        del s, call
        torch.cuda.empty_cache()
    result["prefill_fp8_cache"] = res


def run_head_share(args, result):
    """The share of one of 8 GPUs that split the heads (1 KV head, 6 query heads, its own
    pages): the long prefill (full and SWA layers) and the batch-1 decode and 1M-key verify
    (full layer), at their real per-GPU shapes."""
    import torch

    import synth

    hq, hkv = 6, 1
    share = {}
    for cfg, kind in ((1, "full"), (1, "swa"), (2, "full"), (4, "full")):
        call = synth.make_config(cfg, kind, cache_device="cuda", heads=(hq, hkv))
        s = Staged(call)
        ql = [int(x) for x in call.q_lens]
        kl = [int(x) for x in call.kv_len]
        mode = "prefill" if cfg == 1 else "decode"
        _, per = timed_steps([("kvwrite", s.kvwrite), ("attn", lambda s=s, mode=mode: s.attend(mode))],
                             max(args.steps, 5), args.warmup)
        entry = {"q_heads": hq, "kv_heads": hkv, "attn_ms": round(per["attn"], 4),
                 "kvwrite_ms": round(per["kvwrite"], 4)}
        if mode == "prefill":
            tf = 4 * D * hq * visible_pairs(ql, kl, kind) / (per["attn"] * 1e-3) / 1e12
            entry.update({"tflops": round(tf, 1), "mfma_frac": round(tf / PEAK_BF16_TFLOPS, 4)})
        else:
            nbytes = visible_keys_decode(ql, kl, kind) * 2 * hkv * D * (2 if call.kv_dtype == "bf16" else 1)
            gbs = nbytes / (per["attn"] * 1e-3) / 1e9
            entry.update({"kv_bytes": nbytes, "hbm_gbs": round(gbs, 1), "hbm_frac": round(gbs / PEAK_HBM_GBS, 4)})
        share[f"config{cfg}-{kind}"] = entry
        log(f"  head share config{cfg}-{kind}: {entry}")
        del s, call
        torch.cuda.empty_cache()
    result["head_share_tp8"] = share


def run_projections(args, result, m):
    """The sublayer projections around the attention core at the long-prefill token count:
    packed Q/K/V/gate (5120 -> 14336) and o_proj (6144 -> 5120), y = x W^T in bf16 with
    fp32 accumulation (MFMA-bound at this size)."""
    import torch

    import synth
    from nope_gqa_attention_amd import beamattn as ba

    proj = {}
    for name, n, k in (("qkv_gate", 14336, 5120), ("o_proj", 5120, 6144)):
        x, w = synth.make_linear(m, n, k, [83, n, k], device="cuda")
        y = torch.empty(m, n, dtype=torch.bfloat16, device="cuda")
        _, per = timed_steps([("gemm", lambda: ba.beam_linear_bf16(x, w, y))], args.steps, args.warmup)
        tf = 2.0 * m * n * k / (per["gemm"] * 1e-3) / 1e12
        proj[name] = {"m": m, "n": n, "k": k, "ms": round(per["gemm"], 4), "tflops": round(tf, 1),
                      "mfma_frac": round(tf / PEAK_BF16_TFLOPS, 4)}
        log(f"  projection {name}: {proj[name]}")
        del x, w, y
        torch.cuda.empty_cache()
    result["projections"] = proj


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-rows", type=int, default=256,
                    help="oracle rows sampled per sequence of the long prefill")
    ap.add_argument("--only", choices=("all", "prefill", "decode"), default="all",
                    help="restrict the run (for counter collection); the JSON line needs 'all'")
    ap.add_argument("--summarize-counters", nargs="+", metavar="CSV",
                    help="print the markdown summary of rocprofv3 FETCH_SIZE / WRITE_SIZE counter "
                         "CSVs (no GPU work)")
    ap.add_argument("--summarize-mfma", nargs="+", metavar="CSV",
                    help="print the markdown summary of rocprofv3 MfmaUtil / MfmaFlopsBF16 / "
                         "GRBM_GUI_ACTIVE counter CSVs (no GPU work)")
    ap.add_argument("--summarize-trace", metavar="CSV",
                    help="print the markdown summary of a rocprofv3 kernel-trace CSV (no GPU work)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run one plain 1 GiB device-to-device copy, whose FETCH_SIZE / "
                         "WRITE_SIZE counters calibrate the traffic of the other kernels")
    args = ap.parse_args()
    if args.summarize_counters:
        print(summarize_counters(args.summarize_counters))
        return
    if args.summarize_trace:
        print(summarize_trace(args.summarize_trace))
        return
    if args.summarize_mfma:
        print(summarize_mfma(args.summarize_mfma))
        return
    if args.gpus != 1:
        print(f"bench.py runs on exactly one GPU; --gpus {args.gpus} is not supported "
              "(libbeamattn has no multi-GPU path)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import synth
    from nope_gqa_attention_amd import beamattn as ba

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    ba.load()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    if args.copy_calibration:
        src = torch.ones(1 << 29, dtype=torch.int16, device=dev)     # 1 GiB
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        log("copy calibration: 1 GiB device-to-device copy done")
        del src, dst
    if args.only == "decode":
        args.no_cpu_baseline = True
        result = {"decode": {}}
        run_decode(args, result)
        print(json.dumps(result), flush=True)
        return

    # ---------------------------------------------------------------- prefill workload
    log("generating the long-prefill workload (8 x 2048 new on 98304 cached) ...")
    staged = {}
    for kind in ("full", "swa"):
        call = synth.make_config(1, kind, cache_device="cuda")
        staged[kind] = Staged(call)
        log(f"  {kind}: {call.k_cache.shape[0]} pages staged")
    q_lens = [int(x) for x in staged["full"].call.q_lens]
    kv_lens = [int(x) for x in staged["full"].call.kv_len]
    new_tokens = sum(q_lens)

    parts = []
    for kind in ("full", "swa"):
        s = staged[kind]
        parts.append((f"kvwrite_{kind}", s.kvwrite))
        parts.append((f"prefill_{kind}", lambda s=s: s.attend("prefill")))
    log(f"timing {args.steps} steps after {args.warmup} warmup ...")
    ms_step, per = timed_steps(parts, args.steps, args.warmup)
    flops = {k: 4 * D * HQ * visible_pairs(q_lens, kv_lens, k) for k in ("full", "swa")}
    layers = {}
    for k in ("full", "swa"):
        t_attn = per[f"prefill_{k}"]
        t_kv = per[f"kvwrite_{k}"]
        tf = flops[k] / (t_attn * 1e-3) / 1e12
        kv_bytes = new_tokens * (HQ * D * 2 * 2 + 2 * HKV * D * 2 * 2)   # q in/out, k/v in + cache
        layers[k] = {
            "ms": round(t_attn + t_kv, 4), "prefill_ms": round(t_attn, 4), "kvwrite_ms": round(t_kv, 4),
            "tokens_per_s": round(new_tokens / ((t_attn + t_kv) * 1e-3), 1),
            "prefill_tflops": round(tf, 2), "prefill_mfma_frac": round(tf / PEAK_BF16_TFLOPS, 4),
            "algorithmic_tflop": round(flops[k] / 1e12, 4),
            "kvwrite_gbs": round(kv_bytes / (t_kv * 1e-3) / 1e9, 1),
        }
    dom = layers["full"]
    result = {
        "metric": "attn tokens/s + %roofline (prefill MFMA TFLOP/s, decode HBM GB/s) per layer",
        "value": round(new_tokens / (ms_step * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "long prefill: 8 seqs x 2048 new tokens on 98304 cached, "
                               "NoPE/SSMax full layer + SWA-512 layer, 48/8 heads, d128, "
                               "64-token pages shuffled, bf16 KV",
                   "global_batch": 8, "seq_len": 2048, "cached_tokens": 98304,
                   "parallelism": "none (1 GPU)"},
        "roofline": {"bound": "mfma", "achieved": dom["prefill_tflops"], "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": dom["prefill_mfma_frac"],
                     "traffic": recorded_traffic(),
                     "kernel": "prefill_kernel (full NoPE layer)",
                     "algorithmic_flop_per_launch": flops["full"]},
        "layers": layers,
    }
    log(json.dumps(layers))
    oracle_times = None if args.no_cpu_baseline else {}
    if oracle_times is not None:
        # the oracle on the same bytes, per layer kind, on a bounded sample
        log("timing the fp64 oracle on the host (long prefill, sampled) ...")
        olp = oracle_long_prefill(staged, args.cpu_rows)
        total_s = sum(v["extrapolated_full_s"] for v in olp.values())
        step_s = {k: (layers[k]["ms"]) * 1e-3 for k in layers}
        for k in olp:
            olp[k]["gpu_speedup"] = round(olp[k]["extrapolated_full_s"] / step_s[k], 1)
        result["cpu_baseline"] = {
            "value": round(new_tokens / total_s, 3), "unit": "tokens/s", "cores": oracle_threads(),
            "kind": "oracle",
            "sample": (f"{args.cpu_rows} sampled new tokens per sequence (first, last, page starts, "
                       f"seeded random) of all 8 sequences, on KV head 0 and its 6 query heads, per "
                       f"layer kind (prepare + K/V store of every new token of the sequence, "
                       f"attention over the full visible context, gate); times scaled to all "
                       f"16,384 tokens and 48 heads by visible (row, head, key) triples: "
                       f"extrapolated, measured sample "
                       f"{sum(v['sample_s'] for v in olp.values()):.1f} s"),
            "per_layer": olp,
        }
    del staged, parts
    torch.cuda.empty_cache()

    if not args.no_decode and args.only == "all":  # "--only prefill" skips the decode workloads
        run_tiny_prefill(args, result, oracle_times)
        run_decode(args, result, oracle_times)
        run_prefill_fp8(args, result)
        run_head_share(args, result)
    if args.only in ("all", "prefill"):
        run_projections(args, result, new_tokens)
    if oracle_times is not None:
        result["oracle_timings"] = {"cores": oracle_threads(), "configs": oracle_times}
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
