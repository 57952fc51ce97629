#!/usr/bin/env python3
"""Throughput of the compressed NSA branch on one MI355X.

One step = the whole hot path over one batch of synthetic input resident in
HBM: compress K, compress V (nsa_compress), compressed attention
(nsa_compress_attention_fwd: scores, mask, softmax, P.V) and the importance
scores + top-k (nsa_compress_attention_select, reading the per-row softmax
bias the forward left in the workspace, as nsa_compress_attention does).  W untimed warm-up steps,
then K timed steps bracketed by synchronisations; HIP events recorded on the
launch stream between the four calls give each kernel's duration inside the
same timed region.

Prints one JSON line.  ``value`` is query tokens per second of the whole
step on the batched workload (16 sequences of 8k-32k tokens, 64 query heads
on one KV head); the roofline object is for the dominant kernel (the
attention kernel, bound by MFMA of the element type); ``cpu_baseline`` times
the CPU oracle on the same workload (a seeded sample of its tokens).  Without
``--workload`` the line also carries ``configs``: the same measurement for
every workload (tiny, MQA, GQA varlen, long context, batched), each with its
kernels' fractions of the MFMA and HBM peaks and the oracle timed beside it
(in full where that takes at most --cpu-full-seconds, else sampled).

    python bench.py [--steps K] [--warmup W] [--workload 0..4] [--dtype bf16|f16]
                    [--masks] [--no-cpu-baseline]

``--masks`` passes the workload's causal rules as explicit atten_mask /
topk_mask tensors (the masked entry points: mask packing plus the
every-tile masked kernels) instead of letting the kernels generate them.

``--backward`` times instead the training backward of the compressed branch
on the same workload: the gradients of attention_out (nsa_compress_attention_
backward: query-side and key-side kernels) and of both compressions
(nsa_compress_backward), after one untimed forward.

``--select-attention`` times instead the step that consumes the top-k: the
attention of every query over the raw keys of its selected blocks
(nsa_select_attention), fed with the top-k the compressed branch computes
on the same inputs (computed once, untimed).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "query tokens/sec (compress+attn+topk); TFLOP/s as % of MI355X bf16 MFMA peak"
PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA
PEAK_MFMA_TFLOPS = {"bf16": 2500.0, "f16": 2500.0}   # dense MFMA peak per element type
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E

# HBM bytes of the attention kernel per launch, from rocprofv3 FETCH_SIZE and
# WRITE_SIZE passes scaled by a plain copy of known size.  They are reported
# only while the kernel's sources hash to what they were when counted.
ATTN_SOURCES = ["kv_compression_block_amd/csrc/cmp_attn.hip", "kv_compression_block_amd/csrc/nsa_device.h",
                "kv_compression_block_amd/csrc/nsa_internal.h", "kv_compression_block_amd/csrc/nsa_api.cpp"]
TRAFFIC_RECORD = os.path.join(ROOT, "profiles", "k_cmp_attn_fwd_batched-varlen-B16_hbm.json")


SEL_SOURCES = ["kv_compression_block_amd/csrc/sel_attn.hip", "kv_compression_block_amd/csrc/nsa_device.h",
               "kv_compression_block_amd/csrc/nsa_internal.h", "kv_compression_block_amd/csrc/nsa_api.cpp"]
SEL_TRAFFIC_RECORD = os.path.join(ROOT, "profiles", "k_sel_attn_fwd_batched-varlen-B16_hbm.json")


def attn_source_digest(sources=None) -> str:
    import hashlib
    h = hashlib.sha256()
    for rel in (ATTN_SOURCES if sources is None else sources):
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic(workload: str, record: str = TRAFFIC_RECORD, sources=None):
    """Counted HBM bytes per launch of a kernel, or None when there is no
    count for this workload or the kernel changed since it was taken."""
    try:
        with open(record) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("workload") != workload or rec.get("source_sha256") != attn_source_digest(sources):
        return None
    return float(rec["bytes_per_launch"])


def n_visible(t: np.ndarray, l: int, d: int, n_cmp: int) -> np.ndarray:
    n = np.where(t >= l - 1, (t - l + 1) // d + 1, 0)
    return np.minimum(n, n_cmp)


def workload_work(wl, T2: int) -> dict:
    """Algorithmic work of one step (bookkeeping for the report)."""
    vis = 0
    for T in wl.seqlens:
        nc = (T - wl.l) // wl.d + 1 if T >= wl.l else 0
        vis += int(n_visible(np.arange(T), wl.l, wl.d, nc).sum())
    attn_flops = 2.0 * (wl.D1 + wl.D2) * vis * wl.N1
    comp_flops = 2.0 * wl.l * T2 * wl.N2 * (wl.D1 + wl.D2)
    bytes_ck = 2.0 * (wl.T + T2) * wl.N2 * wl.D1
    bytes_cv = 2.0 * (wl.T + T2) * wl.N2 * wl.D2
    # attention: q, Kc, Vc, out, the two [T, N1, 8] statistics and the
    # per-row bias (4 B) it leaves for the importance pass
    bytes_attn = (2.0 * wl.T * wl.N1 * (wl.D1 + wl.D2) + 2.0 * T2 * wl.N2 * (wl.D1 + wl.D2)
                  + 2 * 32.0 * wl.T * wl.N1 + 4.0 * wl.T * wl.N1)
    # importance + top-k: q, Kc, the per-row bias, topk_indices
    bytes_sel = (2.0 * wl.T * wl.N1 * wl.D1 + 2.0 * T2 * wl.N2 * wl.D1 + 4.0 * wl.T * wl.N1
                 + 4.0 * wl.T * wl.N2 * wl.count)
    return {"visible_pairs": vis, "attn_flops": attn_flops, "compress_flops": comp_flops,
            "bytes_compress_k": bytes_ck, "bytes_compress_v": bytes_cv,
            "bytes_attn": bytes_attn, "bytes_select": bytes_sel}


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(wl, inp, budget_s: float, full_limit_s: float = 60.0) -> dict:
    """The oracle, as it is, on this host's cores: compression of all of K
    and V, then attention/remap/top-k for every token when a pilot run says
    that takes at most ``full_limit_s``, else for a seeded uniform sample of
    tokens sized to ``budget_s`` and scaled to the whole workload."""
    import oracle
    import synth
    import torch
    dt = wl.dtype
    kb, vb, wb = synth.bits(inp["k"]), synth.bits(inp["v"]), synth.bits(inp["w"])
    actq = np.asarray(wl.act_seq_qlen, dtype=np.int64)
    oracle.stage_reset()
    t0 = time.perf_counter()
    kc = oracle.round_to(oracle.compress(kb, wb, actq, wl.l, wl.d, dt), dt)
    vc = oracle.round_to(oracle.compress(vb, wb, actq, wl.l, wl.d, dt), dt)
    t_comp = time.perf_counter() - t0
    actc = oracle.cmp_prefix(wl.seqlens, wl.l, wl.d)
    rng = np.random.default_rng(1234)

    def attn(tokens):
        q_rows = synth.bits(inp["q"][torch.from_numpy(tokens).to(inp["q"].device)])
        t = time.perf_counter()
        oracle.attention(q_rows, tokens, kc, vc, actq, actc, wl.N1, wl.N2, wl.scale, wl.l, wl.d,
                         wl.lsel, wl.count, dtype=dt)
        return time.perf_counter() - t

    # A token's oracle cost grows with the compressed blocks it sees; the
    # pilot's time is scaled by that work, not by its token count.
    cost = np.concatenate([n_visible(np.arange(T), wl.l, wl.d,
                                     (T - wl.l) // wl.d + 1 if T >= wl.l else 0) + 8.0 for T in wl.seqlens])
    pilot = np.sort(rng.choice(wl.T, min(wl.T, 64), replace=False)).astype(np.int64)
    t_pilot = attn(pilot)
    est_full = t_pilot * float(cost.sum()) / float(cost[pilot].sum())
    oracle.stage_reset()
    if est_full <= full_limit_s:
        n = wl.T
        sample = np.arange(wl.T, dtype=np.int64)
    else:
        n = int(min(wl.T, max(32, len(pilot) * max(1.0, budget_s - t_comp) / max(t_pilot, 1e-6))))
        sample = np.sort(rng.choice(wl.T, n, replace=False)).astype(np.int64)
    t_att = attn(sample)
    stages = oracle.stage_seconds()
    est = t_comp + t_att * wl.T / n
    if n == wl.T:
        what = (f"full run: compression of all K/V ({t_comp:.2f} s) + attention/remap/top-k for all "
                f"{wl.T} tokens ({t_att:.2f} s)")
    else:
        what = (f"compression of all K/V ({t_comp:.2f} s) + attention/remap/top-k for {n} of {wl.T} "
                f"tokens drawn uniformly ({t_att:.2f} s), scaled to all tokens (a full run would take "
                f"about {t_att * wl.T / n:.0f} s)")
    scale_att = wl.T / n
    return {"value": wl.T / est, "unit": "query tokens/s", "cores": oracle.threads(), "kind": "oracle",
            "sample": what, "cpu_model": cpu_model(), "host_cpus": os.cpu_count(),
            "seconds_measured": round(t_comp + t_att, 3),
            "stage_seconds_whole_workload": {
                "compress (wall)": round(t_comp, 3),
                **{k + " (thread-s / threads)": round(v * scale_att / max(1, oracle.threads()), 3)
                   for k, v in stages.items() if k != "compress"}},
            "precision": "float64 on the exactly widened element-type inputs"}


def selected_pairs(wl, topk) -> int:
    """Attended (token, key) pairs per KV head, summed: for each token and
    KV head, the keys s <= t of the listed blocks (each block once)."""
    import torch
    total = 0
    s0 = 0
    for T in wl.seqlens:
        S = -(-T // wl.lsel)
        idx = topk[s0:s0 + T].long()                              # [T, N2, count]
        idx, _ = torch.sort(idx, dim=2)
        first = torch.ones_like(idx, dtype=torch.bool)
        first[:, :, 1:] = idx[:, :, 1:] != idx[:, :, :-1]
        valid = first & (idx >= 0) & (idx < S)
        t = torch.arange(T, device=idx.device)[:, None, None]
        keys = torch.clamp(t - idx * wl.lsel + 1, min=0, max=wl.lsel)
        total += int(torch.where(valid, keys, torch.zeros_like(keys)).sum())
        s0 += T
    return total


def select_attention_bench(args, wl, plan, inp, topk, ws, stream) -> dict:
    """Times nsa_select_attention on the workload with the given top-k."""
    import torch
    import kv_compression_block_amd as nsa
    dev = inp["q"].device
    outs = {"attention_out": torch.empty((wl.T, wl.N1, wl.D2), dtype=wl.torch_dtype, device=dev),
            "softmax_lse": torch.empty((wl.T, wl.N1), dtype=torch.float32, device=dev)}

    def run():
        nsa.nsa_select_attention(plan, inp["q"], inp["k"], inp["v"], topk, workspace=ws, outputs=outs,
                                 stream=stream)

    for _ in range(args.warmup):
        run()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    t0 = time.perf_counter()
    for e0, e1 in ev:
        e0.record(stream)
        run()
        e1.record(stream)
    torch.cuda.synchronize()
    ms_step = (time.perf_counter() - t0) * 1e3 / args.steps
    ms_kernel = float(np.mean([e0.elapsed_time(e1) for e0, e1 in ev]))
    pairs = selected_pairs(wl, topk)
    flops = 2.0 * (wl.D1 + wl.D2) * pairs * (wl.N1 // wl.N2)
    tflops = flops / (ms_kernel / 1e3) / 1e12
    peak = PEAK_MFMA_TFLOPS[wl.dtype]
    return {
        "metric": "query tokens/sec (selected-block attention over the top-k blocks)",
        "value": wl.T / (ms_step / 1e3), "unit": "query tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms_step, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": wl.dtype, "data": "synthetic",
        "config": {"workload": wl.name, "B": wl.B, "T": wl.T, "N1": wl.N1, "N2": wl.N2, "D1": wl.D1,
                   "D2": wl.D2, "lsel": wl.lsel, "count": wl.count, "scale": wl.scale, "dtype": wl.dtype,
                   "block_lists": "the compressed branch's top-k on the same inputs",
                   "parallelism": "single-gpu"},
        "roofline": {"kernel": "k_sel_attn_fwd", "bound": "mfma", "achieved": tflops, "peak": peak,
                     "unit": "TFLOP/s", "frac": tflops / peak,
                     "traffic": measured_traffic(wl.name, SEL_TRAFFIC_RECORD, SEL_SOURCES),
                     "traffic_unit": "HBM bytes per launch",
                     "work_per_launch": f"{flops:.4e} flop = 2*(D1+D2) x {pairs} attended (token, key) "
                                        f"pairs per KV head x {wl.N1 // wl.N2} heads per group"},
        "kernels": {"select_attention": {"ms": ms_kernel, "TFLOP/s": tflops}},
        "cpu_baseline": None if args.no_cpu_baseline else select_cpu_baseline(wl, inp, topk, args.cpu_seconds),
    }


def backward_bench(args, wl, plan, inp, kc, vc, outs, stream, T2) -> dict:
    """Times the backward: attention (dq; dkc, dvc) then both compressions."""
    import torch
    import synth
    import kv_compression_block_amd as nsa
    dev = inp["q"].device
    dout = synth.make_output_grad(wl, device=dev, chunk_rows=16384)
    ws = torch.empty(plan.info["backward_workspace_bytes"], dtype=torch.uint8, device=dev)
    grads = {}

    def run(ev=None):
        if ev is not None:
            ev[0].record(stream)
        dq, dk, dv = nsa.nsa_compress_attention_backward(plan, inp["q"], kc, vc, outs["attention_out"], dout,
                                                         outs["softmax_max"], outs["softmax_sum"], workspace=ws,
                                                         stream=stream)
        if ev is not None:
            ev[1].record(stream)
        dxk, dwk = nsa.nsa_compress_backward(inp["k"], inp["w"], dk, wl.act_seq_qlen, wl.l, wl.d, stream=stream)
        dxv, dwv = nsa.nsa_compress_backward(inp["v"], inp["w"], dv, wl.act_seq_qlen, wl.l, wl.d, stream=stream)
        if ev is not None:
            ev[2].record(stream)
        grads.update(dq=dq, dk=dxk, dv=dxv, dw=dwk + dwv)

    for _ in range(args.warmup):
        run()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    t0 = time.perf_counter()
    for ev in evs:
        run(ev)
    torch.cuda.synchronize()
    ms_step = (time.perf_counter() - t0) * 1e3 / args.steps
    ms_attn = float(np.mean([e[0].elapsed_time(e[1]) for e in evs]))
    ms_comp = float(np.mean([e[1].elapsed_time(e[2]) for e in evs]))
    work = workload_work(wl, T2)
    pairs_heads = work["attn_flops"] / (2.0 * (wl.D1 + wl.D2))
    # algorithmic: dV, dP, dq, dK (no recompute of the scores)
    flops = 2.0 * (2 * wl.D1 + 2 * wl.D2) * pairs_heads
    tflops = flops / (ms_attn / 1e3) / 1e12
    peak = PEAK_MFMA_TFLOPS[wl.dtype]
    return {
        "metric": "query tokens/sec (backward of compress+attn)",
        "value": wl.T / (ms_step / 1e3), "unit": "query tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms_step, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": wl.dtype, "data": "synthetic",
        "config": {"workload": wl.name, "B": wl.B, "T": wl.T, "N1": wl.N1, "N2": wl.N2, "D1": wl.D1,
                   "D2": wl.D2, "l": wl.l, "d": wl.d, "dtype": wl.dtype,
                   "gradient": "seeded N(0,1) d_attention_out", "parallelism": "single-gpu"},
        "roofline": {"kernel": "k_cmp_attn_bwd_dq + k_cmp_attn_bwd_dkv", "bound": "mfma", "achieved": tflops,
                     "peak": peak, "unit": "TFLOP/s", "frac": tflops / peak, "traffic": None,
                     "work_per_launch": f"{flops:.4e} flop = 2*(2*D1+2*D2) x {pairs_heads:.4e} visible "
                                        f"(token, block) pairs x heads (dV, dP, dq, dK; the recomputed "
                                        f"scores are not counted)"},
        "kernels": {"attention_backward": {"ms": ms_attn, "TFLOP/s": tflops},
                    "compress_backward_k_and_v": {"ms": ms_comp}},
        "cpu_baseline": None,
    }


def select_cpu_baseline(wl, inp, topk, budget_s: float) -> dict:
    """The oracle's selected-block attention on a bounded uniform sample of
    tokens, scaled to all tokens."""
    import oracle
    import synth
    b = {k: synth.bits(inp[k]) for k in ("q", "k", "v")}
    tk = topk.cpu().numpy()
    rng = np.random.default_rng(4321)

    def run(tokens):
        t = time.perf_counter()
        oracle.select_attention(b["q"], b["k"], b["v"], tk, wl.act_seq_qlen, wl.N1, wl.N2, wl.scale,
                                wl.lsel, tokens=tokens, dtype=wl.dtype)
        return time.perf_counter() - t

    pilot = np.sort(rng.choice(wl.T, 64, replace=False)).astype(np.int64)
    tp = run(pilot)
    n = int(min(wl.T, max(64, 64 * budget_s / max(tp, 1e-6))))
    sample = np.sort(rng.choice(wl.T, n, replace=False)).astype(np.int64)
    ts = run(sample)
    return {"value": n / ts, "unit": "query tokens/s", "cores": oracle.threads(), "kind": "oracle",
            "sample": f"selected-block attention for {n} of {wl.T} tokens drawn uniformly ({ts:.2f} s)",
            "seconds_measured": round(tp + ts, 3)}


class Path:
    """Inputs, plan, outputs and workspace of one workload, resident on the GPU."""

    def __init__(self, args, wl, dev, masks_on: bool = False, split_tiles: int = 0):
        import torch
        import synth
        import kv_compression_block_amd as nsa
        self.wl, self.dev, self.split_tiles = wl, dev, split_tiles
        print(f"[bench] workload {wl.name}: generating inputs", file=sys.stderr, flush=True)
        self.inp = synth.make_inputs(wl, device=dev, chunk_rows=16384)
        c_pre, s_pre, pc, ps = [], [], 0, 0
        for T in wl.seqlens:
            pc += nsa.nsa_compress_out_len(T, wl.l, wl.d)
            ps += -(-T // wl.lsel)
            c_pre.append(pc)
            s_pre.append(ps)
        self.T2 = pc
        self.plan = nsa.nsa_compress_attention_get_workspace(wl.act_seq_qlen, c_pre, s_pre, wl.N1, wl.N2,
                                                             wl.D1, wl.D2, wl.scale, wl.l, wl.d, wl.lsel,
                                                             wl.count, wl.torch_dtype)
        self.kc = torch.empty((pc, wl.N2, wl.D1), dtype=wl.torch_dtype, device=dev)
        self.vc = torch.empty((pc, wl.N2, wl.D2), dtype=wl.torch_dtype, device=dev)
        self.outs = {"attention_out": torch.empty((wl.T, wl.N1, wl.D2), dtype=wl.torch_dtype, device=dev),
                     "topk_indices": torch.empty((wl.T, wl.N2, wl.count), dtype=torch.int32, device=dev),
                     "softmax_max": torch.empty((wl.T, wl.N1, 8), dtype=torch.float32, device=dev),
                     "softmax_sum": torch.empty((wl.T, wl.N1, 8), dtype=torch.float32, device=dev)}
        self.masks = {}
        if masks_on:
            # The positional rules spelled out as masks (True = masked out), one
            # matrix for all sequences: rows = local query positions.
            t_max = max(wl.seqlens)
            t = torch.arange(t_max, device=dev)[:, None]
            ncm = max(nsa.nsa_compress_out_len(T, wl.l, wl.d) for T in wl.seqlens)
            self.masks["atten_mask"] = (torch.arange(ncm, device=dev)[None, :] * wl.d + wl.l - 1) > t
            self.masks["topk_mask"] = (torch.arange(max(-(-T // wl.lsel) for T in wl.seqlens),
                                                    device=dev)[None, :] * wl.lsel) > t
        ws_bytes = self.plan.info["masked_workspace_bytes"] if masks_on else self.plan.workspace_bytes
        if split_tiles:
            ws_bytes = max(ws_bytes, nsa.nsa_compress_attention_split_workspace(self.plan, split_tiles))
        self.ws = torch.empty((max(ws_bytes, 1),), dtype=torch.uint8, device=dev)
        self.stream = torch.cuda.current_stream(dev)

    def step(self, ev=None):
        """One pass of the hot path; events (if given) bracket each call."""
        import kv_compression_block_amd as nsa
        wl, inp, stream, outs = self.wl, self.inp, self.stream, self.outs
        if ev is not None:
            ev[0].record(stream)
        nsa.nsa_compress(inp["k"], inp["w"], wl.act_seq_qlen, wl.l, wl.d, out=self.kc, stream=stream)
        if ev is not None:
            ev[1].record(stream)
        nsa.nsa_compress(inp["v"], inp["w"], wl.act_seq_qlen, wl.l, wl.d, out=self.vc, stream=stream)
        if ev is not None:
            ev[2].record(stream)
        if self.split_tiles:
            nsa.nsa_compress_attention_fwd_split(self.plan, inp["q"], self.kc, self.vc, self.split_tiles,
                                                 workspace=self.ws, outputs=outs, stream=stream)
        else:
            nsa.nsa_compress_attention_fwd(self.plan, inp["q"], self.kc, self.vc, workspace=self.ws, outputs=outs,
                                           stream=stream, atten_mask=self.masks.get("atten_mask"))
        if ev is not None:
            ev[3].record(stream)
        # the row statistics from the per-row bias the forward left in the
        # workspace (as nsa_compress_attention does)
        nsa.nsa_compress_attention_select(self.plan, inp["q"], self.kc, None, None,
                                          workspace=self.ws, outputs=outs, stream=stream,
                                          atten_mask=self.masks.get("atten_mask"),
                                          topk_mask=self.masks.get("topk_mask"))
        if ev is not None:
            ev[4].record(stream)

    def time_steps(self, steps: int, warmup: int) -> dict:
        """W untimed steps, then K timed steps between synchronisations; HIP
        events on the launch stream give each call's duration."""
        import torch
        wl = self.wl
        print(f"[bench] {wl.name}: warmup {warmup} steps", file=sys.stderr, flush=True)
        for _ in range(warmup):
            self.step()
        torch.cuda.synchronize()
        events = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(steps)]
        print(f"[bench] {wl.name}: timing {steps} steps", file=sys.stderr, flush=True)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(steps):
            self.step(events[i])
        torch.cuda.synchronize()
        ms_step = (time.perf_counter() - t0) * 1e3 / steps
        names = ["compress_k", "compress_v", "attention", "select_topk"]
        per = {n: float(np.mean([events[i][j].elapsed_time(events[i][j + 1]) for i in range(steps)]))
               for j, n in enumerate(names)}
        work = workload_work(wl, self.T2)
        peak = PEAK_MFMA_TFLOPS[wl.dtype]
        attn_tflops = work["attn_flops"] / (per["attention"] / 1e3) / 1e12
        # attainable attention rate on the roofline: min(MFMA peak, intensity x HBM peak)
        ai = work["attn_flops"] / work["bytes_attn"]
        attainable = min(peak, ai * PEAK_HBM_GBS / 1e3)
        recompute = 2.0 * wl.D1 * work["visible_pairs"] * wl.N1
        # The importance pass is bound by arithmetic, not bytes: the recomputed
        # Q.K^T on MFMA, and per score an FMA, an exp2 (half rate) and an add on
        # the vector ALUs (four wave64 issue slots of 4 cycles per 64 scores,
        # 1024 SIMDs at 2.4 GHz).  On this part the two pipes barely overlap,
        # so the floor it can reach is their sum.
        sel_mfma_ms = recompute / (peak * 1e12) * 1e3
        sel_valu_ms = work["visible_pairs"] * wl.N1 * 0.25 / (1024 * 2.4e9) * 1e3

        def gbs(b, ms):
            return b / (ms / 1e3) / 1e9

        kernels = {
            "compress_k": {"ms": per["compress_k"], "GB/s": gbs(work["bytes_compress_k"], per["compress_k"]),
                           "frac_of_hbm_peak": gbs(work["bytes_compress_k"], per["compress_k"]) / PEAK_HBM_GBS},
            "compress_v": {"ms": per["compress_v"], "GB/s": gbs(work["bytes_compress_v"], per["compress_v"]),
                           "frac_of_hbm_peak": gbs(work["bytes_compress_v"], per["compress_v"]) / PEAK_HBM_GBS},
            "attention": {"ms": per["attention"], "TFLOP/s": attn_tflops, "mfma_frac": attn_tflops / peak,
                          "flop_per_byte": ai, "attainable_TFLOP/s": attainable,
                          "frac_of_attainable": attn_tflops / attainable},
            "select_topk": {"ms": per["select_topk"], "GB/s": gbs(work["bytes_select"], per["select_topk"]),
                            "frac_of_hbm_peak": gbs(work["bytes_select"], per["select_topk"]) / PEAK_HBM_GBS,
                            "recompute_TFLOP/s": recompute / (per["select_topk"] / 1e3) / 1e12,
                            "alu_floor_ms": {"mfma": sel_mfma_ms, "valu": sel_valu_ms},
                            "frac_of_serial_alu_floor": (sel_mfma_ms + sel_valu_ms) / per["select_topk"]},
        }
        total_flops = work["attn_flops"] + work["compress_flops"]
        return {"ms_per_step": ms_step, "query_tokens_per_s": wl.T / (ms_step / 1e3),
                "tflops_algorithmic": total_flops / (ms_step / 1e3) / 1e12,
                "frac_of_bf16_peak": total_flops / (ms_step / 1e3) / 1e12 / PEAK_BF16_TFLOPS,
                "kernels": kernels, "work": work}

    def close(self):
        self.plan.destroy()


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", type=int, default=None, choices=range(5),
                    help="measure only this workload (default: the batched workload as the headline, "
                         "then every other workload)")
    ap.add_argument("--dtype", default="bf16", choices=["bf16", "f16"],
                    help="element type of q, k, v and the weight (default bf16)")
    ap.add_argument("--masks", action="store_true",
                    help="give the causal rules as explicit atten_mask / topk_mask tensors")
    ap.add_argument("--select-attention", action="store_true",
                    help="time the selected-block attention over the compressed branch's top-k")
    ap.add_argument("--backward", action="store_true",
                    help="time the backward of the compressed attention and of the compression")
    ap.add_argument("--split-tiles", type=int, default=0,
                    help="run the attention as the split launch, pieces of at most this many key tiles")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="budget of a sampled oracle run (workloads whose full run takes longer than "
                         "--cpu-full-seconds)")
    ap.add_argument("--cpu-full-seconds", type=float, default=60.0)
    ap.add_argument("--copy-bytes", type=int, default=0,
                    help="only run a plain device copy of this many bytes (calibrates the HBM byte "
                         "counters against a kernel of known traffic) and exit")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: the path runs on a single MI355X and this build has no "
              f"multi-GPU leg (asked for --gpus {args.gpus}).", file=sys.stderr)
        return 2

    import torch
    import synth
    from kv_compression_block_amd import _lib

    if not os.path.exists(_lib.LIB_PATH):
        from kv_compression_block_amd import build as _build
        _build.build()
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.copy_bytes:
        src = torch.ones(args.copy_bytes, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        dst.copy_(src)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1)
        print(json.dumps({"copy_bytes": args.copy_bytes, "read_bytes": args.copy_bytes,
                          "write_bytes": args.copy_bytes, "ms": ms,
                          "GB/s": 2 * args.copy_bytes / (ms / 1e3) / 1e9}), flush=True)
        return 0
    head_id = 4 if args.workload is None else args.workload
    wl = synth.WORKLOADS[head_id].with_dtype(args.dtype)
    if args.split_tiles and args.masks:
        raise SystemExit("--split-tiles applies to the positional rule only")
    path = Path(args, wl, dev, masks_on=args.masks, split_tiles=args.split_tiles)

    if args.backward or args.select_attention:
        path.step()
        torch.cuda.synchronize()
        if args.backward:
            res = backward_bench(args, wl, path.plan, path.inp, path.kc, path.vc, path.outs, path.stream, path.T2)
        else:
            res = select_attention_bench(args, wl, path.plan, path.inp, path.outs["topk_indices"], path.ws,
                                         path.stream)
        path.close()
        print(json.dumps(res), flush=True)
        return 0

    m = path.time_steps(args.steps, args.warmup)
    work, kernels = m.pop("work"), m["kernels"]
    peak = PEAK_MFMA_TFLOPS[wl.dtype]
    attn_tflops = kernels["attention"]["TFLOP/s"]
    res = {
        "metric": METRIC,
        "value": m["query_tokens_per_s"],
        "unit": "query tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": m["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype,
        "data": "synthetic",
        "config": {"workload": wl.name, "B": wl.B, "T": wl.T, "N1": wl.N1, "N2": wl.N2, "D1": wl.D1,
                   "D2": wl.D2, "l": wl.l, "d": wl.d, "lsel": wl.lsel, "count": wl.count,
                   "scale": wl.scale, "dtype": wl.dtype,
                   "masks": "explicit tensors (the causal rules spelled out)" if args.masks else "positional rules",
                   "attention_launch": (f"split key ranges, at most {args.split_tiles} tiles of 32 blocks per piece"
                                        if args.split_tiles else "single pass"),
                   "parallelism": "single-gpu"},
        "tflops_algorithmic": m["tflops_algorithmic"],
        "frac_of_bf16_peak": m["frac_of_bf16_peak"],
        "roofline": {"kernel": "k_cmp_attn_fwd", "bound": "mfma", "achieved": attn_tflops,
                     "peak": peak, "unit": "TFLOP/s", "frac": attn_tflops / peak,
                     "traffic": None if (args.masks or args.split_tiles) else measured_traffic(wl.name),
                     "traffic_unit": "HBM bytes per launch",
                     "work_per_launch": f"{work['attn_flops']:.4e} flop = 2*(D1+D2) x {work['visible_pairs']} "
                                        f"visible (token, block) pairs x {wl.N1} heads"},
        "kernels": kernels,
    }
    if args.masks:
        res["kernels_note"] = ("with --masks, 'attention' includes packing atten_mask and 'select_topk' "
                               "includes packing both masks (each call packs what it reads)")
    if not args.no_cpu_baseline:
        print(f"[bench] {wl.name}: CPU oracle baseline", file=sys.stderr, flush=True)
        res["cpu_baseline"] = cpu_baseline(wl, path.inp, args.cpu_seconds, args.cpu_full_seconds)
    else:
        res["cpu_baseline"] = None
    path.close()
    del path
    torch.cuda.empty_cache()

    if args.workload is None:
        # Every other workload, measured the same way (same step, same timing);
        # the headline above is the batched workload.
        configs = {wl.name: {"ms_per_step": m["ms_per_step"], "query_tokens_per_s": m["query_tokens_per_s"],
                             "tflops_algorithmic": m["tflops_algorithmic"], "kernels": kernels,
                             "cpu_baseline": res["cpu_baseline"]}}
        for wid in (0, 1, 2, 3):
            w = synth.WORKLOADS[wid].with_dtype(args.dtype)
            p = Path(args, w, dev, masks_on=args.masks, split_tiles=args.split_tiles)
            mw = p.time_steps(max(args.steps, 200) if wid == 0 else args.steps, args.warmup)
            mw.pop("work")
            if not args.no_cpu_baseline:
                print(f"[bench] {w.name}: CPU oracle baseline", file=sys.stderr, flush=True)
                mw["cpu_baseline"] = cpu_baseline(w, p.inp, args.cpu_seconds, args.cpu_full_seconds)
            p.close()
            del p
            torch.cuda.empty_cache()
            configs[w.name] = mw
        res["configs"] = configs
    print(json.dumps(res), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
