"""Throughput of the fused attention forward + backward on one MI355X.

One step = the whole hot path on one batch of seeded synthetic input already
resident in HBM: attn_fwd, attn_bwd_preprocess, attn_bwd (plus the dQ sum on
the split path) and attn_bwd_postprocess, all through the C ABI.

Prints one JSON line.  ``value`` is fwd+bwd TFLOP/s with the FLOP count
4*B*Hq*S^2*D (forward) + 10*B*Hq*S^2*D (backward), halved under causal
masking.  ``roofline`` covers the dominant kernel (the backward kernel),
timed with HIP events on the stream it runs on; ``cpu_baseline`` times the
fp64 oracle on the host cores on a bounded sample of the same workload.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0  # MI355X HBM3E
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
METRIC = "attention fwd+bwd TFLOP/s (bf16, causal) and % of MI355X bf16 MFMA peak"
DEFAULT_WORKLOAD = "mha_causal_b4_h32_s4096_d128"


def flops(w, causal):
    f = w.batch * w.heads_q * w.seqlen * w.seqlen * w.head_dim
    div = 2 if causal else 1
    return 4 * f / div, 10 * f / div


BWD_SOURCES = ("bwd.hip", "common.h", "kernels.h")  # what the backward kernel is built from
GLA_SOURCES = ("gla.hip", "common.h", "kernels.h")  # what the GLA chunk backward is built from
SMLA_SOURCES = ("smla.hip", "smla_split.hip", "smla_split.h", "common.h", "kernels.h")  # ... the sparse MLA kernels
MERGE_SOURCES = ("merge.hip", "common.h", "kernels.h")  # ... the partial-merge kernel


def kernel_source_hash(sources=BWD_SOURCES):
    """Hash of a kernel's sources: recorded counters stay valid until one of
    these files changes."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "attention_backward_fwd_amd", "csrc")
    for name in sources:
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode() + f.read())
    return h.hexdigest()[:16]


def recorded_traffic(workload, path, sources=BWD_SOURCES):
    """HBM bytes per launch from the committed counter summary, if it still
    describes the current kernel sources; else None."""
    fn = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(fn) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    entry = rec.get(f"{workload}/{path}")
    if not entry or entry.get("source_hash") != kernel_source_hash(sources):
        return None
    return entry.get("bytes_per_launch")


def recorded_util(workload, path, sources=BWD_SOURCES):
    """Matrix-core utilisation of the backward kernel from the committed
    counter summary (SQ_VALU_MFMA_BUSY_CYCLES over the XCD-average clock's
    cycles x 1024 SIMDs), if it still describes the current kernel sources;
    else None.  Unlike `frac`, it does not depend on the clock the GPU ran at."""
    fn = os.path.join(ROOT, "profiles", "mfma_util.json")
    try:
        with open(fn) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    entry = rec.get(f"{workload}/{path}")
    if not entry or entry.get("source_hash") != kernel_source_hash(sources):
        return None
    return entry


def _blas_threads():
    try:
        from threadpoolctl import threadpool_info
        return max((i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"), default=1)
    except Exception:  # threadpoolctl missing: numpy BLAS default
        return os.cpu_count() or 1


def cpu_baseline(w, causal, budget_s):
    """The fp64 oracle on host cores, one KV group at a time until the budget is used."""
    import numpy as np
    import torch

    from attention_backward_fwd_amd.synthetic import make_inputs
    from oracle import attention as orc

    cores = _blas_threads()
    g = w.groups
    groups_done, t_total = 0, 0.0
    seed = 0
    while t_total < budget_s and groups_done < w.batch * (w.heads_q // g):
        # one (batch, KV head) group: g query heads and their KV head, full length
        inp = make_inputs(1, w.seqlen, g, 1, w.head_dim, seed=seed + groups_done, qk_mult=w.qk_mult)
        f = {n: t.to(torch.float64).numpy() for n, t in inp.items()}
        t0 = time.perf_counter()
        orc.attention_fwd(f["q"], f["k"], f["v"], w.scale, causal, g)
        orc.attention_bwd(f["q"], f["k"], f["v"], f["do"], w.scale, causal, g)
        t_total += time.perf_counter() - t0
        groups_done += 1
    fwd_f, bwd_f = flops(w, causal)
    frac = groups_done * g / (w.batch * w.heads_q)
    tflops = (fwd_f + bwd_f) * frac / t_total / 1e12
    return {"value": round(tflops, 6), "unit": "TFLOP/s", "cores": int(cores), "kind": "oracle",
            "sample": f"{groups_done} of {w.batch * (w.heads_q // g)} (batch, KV-head) groups at full length "
                      f"({groups_done * g} query heads), fwd+bwd in fp64, {t_total:.1f} s; "
                      f"FLOPs counted with the same causal-halved formula"}


def bench_merge(args, w, bd, torch):
    """attn_merge of P synthetic partials shaped like the workload's O/LSE:
    one JSON line with GB/s against the HBM peak (bytes = every part's O
    and LSE read once, O and LSE written once)."""
    n = args.merge_parts
    g = torch.Generator(device="cuda:0").manual_seed(7)
    o_p = torch.randn((n, w.batch, w.seqlen, w.heads_q, w.head_dim), device="cuda:0", generator=g).to(torch.bfloat16)
    l_p = torch.randn((n, w.batch, w.heads_q, w.seqlen), device="cuda:0", generator=g)
    shape = bd.make_shape(w.batch, w.seqlen, w.heads_q, 1, w.head_dim)
    o = torch.empty(o_p.shape[1:], dtype=torch.bfloat16, device="cuda:0")
    lse = torch.empty(l_p.shape[1:], dtype=torch.float32, device="cuda:0")
    stream = torch.cuda.current_stream()
    for _ in range(args.warmup):
        bd.attn_merge(o_p, l_p, n, o, lse, shape, stream)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2 * args.steps)]
    torch.cuda.synchronize()
    for i in range(args.steps):
        ev[2 * i].record(stream)
        bd.attn_merge(o_p, l_p, n, o, lse, shape, stream)
        ev[2 * i + 1].record(stream)
    torch.cuda.synchronize()
    ms = sum(ev[2 * i].elapsed_time(ev[2 * i + 1]) for i in range(args.steps)) / args.steps
    nq = w.batch * w.seqlen * w.heads_q * w.head_dim
    rows = w.batch * w.heads_q * w.seqlen
    nbytes = n * (2 * nq + 4 * rows) + 2 * nq + 4 * rows
    gbs = nbytes / (ms * 1e-3) / 1e9
    cpu = None
    if not args.no_cpu_baseline:
        from oracle import cp
        bsl = 1  # one batch element of the partials
        op_ = o_p[:, :bsl].float().cpu().double().numpy()
        lp_ = l_p[:, :bsl].cpu().double().numpy()
        t1 = time.perf_counter()
        cp.merge_partials(op_, lp_)
        t_cpu = time.perf_counter() - t1
        cpu = {"value": round(nbytes * bsl / w.batch / t_cpu / 1e9, 4), "unit": "GB/s", "cores": int(_blas_threads()),
               "kind": "oracle", "sample": f"batch element 0 of {w.batch} ({n} parts), fp64, {t_cpu:.1f} s; "
                                           f"the same bytes per row"}
    print(json.dumps({"metric": "attn_merge HBM throughput", "value": round(gbs, 1), "unit": "GB/s",
                      "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
                      "higher_is_better": True, "dtype": "bf16 O, fp32 LSE", "data": "synthetic",
                      "config": {"workload": w.name, "parts": n},
                      "roofline": {"kernel": "merge_kernel", "bound": "hbm", "achieved": round(gbs, 1),
                                   "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4),
                                   "traffic": recorded_traffic(w.name, f"merge{n}", MERGE_SOURCES)},
                      **({"cpu_baseline": cpu} if cpu else {})}), flush=True)


def bench_varlen(args, bd, torch):
    """The whole step over the packed causal pack of sequences: attn_fwd_varlen,
    the preprocess, attn_bwd_varlen (plus the dQ sum on the split path) and
    attn_bwd_varlen_postprocess.  FLOPs are the per-sequence causal-halved counts summed
    over the pack; padding rows count nothing."""
    from attention_backward_fwd_amd.synthetic import VARLEN_PACK, varlen_pack_inputs

    spec = VARLEN_PACK
    inp, lengths, cu_cpu = varlen_pack_inputs(spec)
    dev = torch.device("cuda:0")
    d = {n: t.to(dev) for n, t in inp.items()}
    cu = cu_cpu.to(dev)
    q, k, v, do = d["q"], d["k"], d["v"], d["do"]
    hq, dim = spec["heads_q"], spec["head_dim"]
    scale = 1.0 / math.sqrt(dim)
    use_atomic = args.use_atomic
    m = max(lengths)
    sh = bd.varlen_shape_of(q, k, len(lengths), m)
    o = torch.empty_like(q)
    lse = torch.empty((hq, q.shape[0]), dtype=torch.float32, device=dev)
    bb = bd.VarlenBwdBuffers(q, k, len(lengths), m, True, use_atomic)
    stream = torch.cuda.current_stream()
    ev = {n: [torch.cuda.Event(enable_timing=True) for _ in range(2 * args.steps)] for n in ("fwd", "bwd")}

    def step(i=None):
        if i is not None:
            ev["fwd"][2 * i].record(stream)
        bd.attn_fwd_varlen(q, k, v, o, lse, cu, cu, sh, scale, True, stream)
        if i is not None:
            ev["fwd"][2 * i + 1].record(stream)
        bd.attn_bwd_preprocess(o, do, bb.delta, bb.dq_accum if use_atomic else None, bb.dense, stream)
        if i is not None:
            ev["bwd"][2 * i].record(stream)
        bd.attn_bwd_varlen(q, k, v, do, lse, bb.delta, bb.dq_accum, bb.dk, bb.dv, bb.workspace, cu, cu, sh,
                           scale, True, use_atomic, stream)
        if i is not None:
            ev["bwd"][2 * i + 1].record(stream)
        bd.attn_bwd_varlen_postprocess(bb.dq_accum, bb.workspace, bb.dq, bb.dk, bb.dv, sh, stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    per = sum(n * n for n in lengths) * hq * dim / 2  # causal
    fwd_f, bwd_f = 4 * per, 10 * per
    fwd_ms = sum(ev["fwd"][2 * i].elapsed_time(ev["fwd"][2 * i + 1]) for i in range(args.steps)) / args.steps
    bwd_ms = sum(ev["bwd"][2 * i].elapsed_time(ev["bwd"][2 * i + 1]) for i in range(args.steps)) / args.steps
    value = (fwd_f + bwd_f) * args.steps / elapsed / 1e12
    bwd_tflops = bwd_f / (bwd_ms * 1e-3) / 1e12
    path = "atomic" if use_atomic else "split"
    cpu = None
    if not args.no_cpu_baseline:
        from oracle import varlen as vl
        f = {n: x.to(torch.float64).numpy() for n, x in inp.items()}
        cul = cu_cpu.tolist()
        done, flop_done, t_cpu = 0, 0.0, 0.0
        for a, e in zip(cul[:-1], cul[1:]):  # whole sequences, all heads, in pack order
            if t_cpu >= args.cpu_budget:
                break
            t1 = time.perf_counter()
            vl.varlen_bwd(f["q"][a:e], f["k"][a:e], f["v"][a:e], f["do"][a:e], [0, e - a], scale, True, 1)
            t_cpu += time.perf_counter() - t1
            done += 1
            flop_done += 14 * (e - a) ** 2 * hq * dim / 2
        cpu = {"value": round(flop_done / t_cpu / 1e12, 6), "unit": "TFLOP/s", "cores": int(_blas_threads()),
               "kind": "oracle", "sample": f"{done} of {len(lengths)} sequences (all heads), fwd+bwd in fp64, "
                                           f"{t_cpu:.1f} s; the same per-sequence causal FLOP count"}
    print(json.dumps({
        "metric": "packed-sequence attention fwd+bwd TFLOP/s (bf16, causal)", "value": round(value, 3),
        "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(elapsed / args.steps * 1e3, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": spec["name"], "lengths": lengths, "padding_rows": spec["pad"], "heads_q": hq,
                   "heads_kv": spec["heads_kv"], "head_dim": dim, "causal": True, "dq_path": path},
        "pct_of_peak": round(100.0 * value / PEAK_BF16_TFLOPS, 3),
        "fwd_kernel_ms": round(fwd_ms, 4), "fwd_tflops": round(fwd_f / (fwd_ms * 1e-3) / 1e12, 3),
        "bwd_kernel_ms": round(bwd_ms, 4),
        "roofline": {"kernel": "bwd_kernel (packed)" + ("" if use_atomic else " + dq_sum_varlen_kernel"),
                     "bound": "mfma", "achieved": round(bwd_tflops, 3), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(bwd_tflops / PEAK_BF16_TFLOPS, 4),
                     "traffic": recorded_traffic(spec["name"], path)},
        **({"cpu_baseline": cpu} if cpu else {}),
    }), flush=True)


def bench_gla(args, bd, torch):
    """Simple gated linear attention, chunked backward (gla_chunk_bwd: the two
    chunk sweeps with on-chip state, then the gate's running sum) on the GLA
    workload.
    HBM-bound: ``value`` is the algorithmic bytes (q, k, v, do, g read once;
    dq, dk, dv, dg written once) per second of the whole call."""
    from attention_backward_fwd_amd.synthetic import GLA_WORKLOAD, gla_inputs

    w = GLA_WORKLOAD
    b, t, h, d = w["batch"], w["seqlen"], w["heads"], w["head_dim"]
    dev = torch.device("cuda:0")
    inp = {n: x.to(dev) for n, x in gla_inputs(b, t, h, d, seed=0).items()}
    scale = 1.0 / math.sqrt(d)
    bb = bd.GlaBuffers(inp["q"])
    stream = torch.cuda.current_stream()

    def call():
        bd.gla_chunk_bwd(inp["q"], inp["k"], inp["v"], inp["g"], inp["do"], bb.dq, bb.dk, bb.dv, bb.dg,
                         bb.workspace, bb.shape, scale, stream)

    for _ in range(args.warmup):
        call()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2 * args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        ev[2 * i].record(stream)
        call()
        ev[2 * i + 1].record(stream)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms = sum(ev[2 * i].elapsed_time(ev[2 * i + 1]) for i in range(args.steps)) / args.steps
    n_elem = b * t * h * d
    nbytes = 4 * n_elem * 2 + b * t * h * 4 + 3 * n_elem * 2 + b * t * h * 4
    n_chunks = b * h * ((t + 63) // 64)
    flop = n_chunks * (10 * 64 * d * d + 10 * 64 * 64 * d)  # the chunked algorithm's matrix products
    gbs = nbytes / (ms * 1e-3) / 1e9
    cpu = None
    if not args.no_cpu_baseline:
        from oracle import linear_attn as la
        f = {n: x.cpu().to(torch.float64).numpy() for n, x in inp.items()}
        heads, t_cpu = 0, 0.0
        while t_cpu < args.cpu_budget and heads < b * h:
            bb_, hh = divmod(heads, h)
            t1 = time.perf_counter()
            la.gla_bwd(f["q"][bb_:bb_ + 1], f["k"][bb_:bb_ + 1], f["v"][bb_:bb_ + 1], f["g"][bb_:bb_ + 1],
                       f["do"][bb_:bb_ + 1], scale, heads=[(0, hh)])
            t_cpu += time.perf_counter() - t1
            heads += 1
        cpu = {"value": round(nbytes * heads / (b * h) / t_cpu / 1e9, 4), "unit": "GB/s", "cores": int(_blas_threads()),
               "kind": "oracle", "sample": f"{heads} of {b * h} (batch, head) pairs at full length, quadratic fp64 "
                                           f"form, {t_cpu:.1f} s; the same algorithmic bytes per head"}
    print(json.dumps({
        "metric": "simple-GLA chunk backward throughput (algorithmic HBM bytes)", "value": round(gbs, 1),
        "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(elapsed / args.steps * 1e3, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16 (fp32 accumulation, fp32 gate)", "data": "synthetic",
        "config": {"workload": w["name"], "batch": b, "seq_len": t, "heads": h, "head_dim": d, "chunk": 64},
        "bwd_ms": round(ms, 4), "tokens_per_s": round(b * t / (ms * 1e-3), 1),
        "mfma_tflops": round(flop / (ms * 1e-3) / 1e12, 3),
        "roofline": {"kernel": "gla_sweep + gla_dg", "bound": "hbm", "achieved": round(gbs, 1),
                     "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4),
                     "traffic": recorded_traffic(w["name"], "chunk_bwd", GLA_SOURCES)},
        **({"cpu_baseline": cpu} if cpu else {}),
    }), flush=True)


def bench_smla(args, bd, torch):
    """Sparse MLA forward + backward on the sparse MLA workload.  FLOPs: per
    (token, head, valid entry) 2*(576 + 512) forward and
    2*(576 + 512 + 576 + 576 + 512) backward (S, dP, dQ, dK, dV).  Two dKV
    paths: fp32 atomic adds (576 per token, valid entry and 32-head tile;
    ``atomics`` reports their rate), then a postprocess cast; or the
    deterministic path (--use-atomic 0): index sort, per-entry partial rows,
    fixed-order sum, all inside one call.  The path not chosen is timed after
    it on the same inputs (``other_path``) unless --no-other-path."""
    from attention_backward_fwd_amd.synthetic import SMLA_WORKLOAD, smla_indices, smla_inputs

    w = SMLA_WORKLOAD
    t, h, k = w["tokens"], w["heads"], w["topk"]
    dev = torch.device("cuda:0")
    inp = {n: x.to(dev) for n, x in smla_inputs(t, t, h, seed=0).items()}
    idx_cpu = smla_indices(t, t, k, seed=0)
    idx = idx_cpu.to(dev)
    scale = 1.0 / math.sqrt(576)
    q, kv, do = inp["q"], inp["kv"], inp["do"]
    shape = bd.smla_shape_of(q, kv, idx)
    o = torch.empty((t, h, 512), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((t, h), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()
    n_valid = int((idx_cpu >= 0).sum())
    fwd_f = 2.0 * n_valid * h * (576 + 512)
    bwd_f = 2.0 * n_valid * h * (576 + 512 + 576 + 576 + 512)

    def run(use_atomic, steps, warmup):
        bb = bd.SmlaBwdBuffers(q, kv, use_atomic, idx)
        names = ("fwd", "pre", "call", "post")
        ev = {n: [torch.cuda.Event(enable_timing=True) for _ in range(2 * steps)] for n in names}

        def mark(n, i, end):
            if i is not None:
                ev[n][2 * i + end].record(stream)

        def step(i=None):
            mark("fwd", i, 0)
            bd.attn_sparse_mla_fwd(q, kv, idx, o, lse, shape, scale, stream)
            mark("fwd", i, 1)
            mark("pre", i, 0)
            bd.attn_sparse_mla_bwd_preprocess(o, do, bb.delta, bb.dkv_accum, shape, stream)
            mark("pre", i, 1)
            mark("call", i, 0)
            if use_atomic:
                bd.attn_sparse_mla_bwd(q, kv, do, idx, lse, bb.delta, bb.dq, bb.dkv_accum, shape, scale, stream)
            else:
                bd.attn_sparse_mla_bwd_split(q, kv, do, idx, lse, bb.delta, bb.dq, bb.dkv, bb.workspace, shape, scale,
                                             stream)
            mark("call", i, 1)
            mark("post", i, 0)
            if use_atomic:
                bd.attn_sparse_mla_bwd_postprocess(bb.dkv_accum, bb.dkv, shape, stream)
            mark("post", i, 1)

        for _ in range(warmup):
            step()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(steps):
            step(i)
        torch.cuda.synchronize()
        elapsed = time.perf_counter() - t0
        ms = {n: sum(ev[n][2 * i].elapsed_time(ev[n][2 * i + 1]) for i in range(steps)) / steps for n in names}
        ms["backward"] = ms["pre"] + ms["call"] + ms["post"]
        ws = 0 if bb.workspace is None else bb.workspace.numel()
        del bb
        return ms, elapsed, ws

    use_atomic = bool(args.use_atomic)
    ms, elapsed, ws = run(use_atomic, args.steps, args.warmup)
    value = (fwd_f + bwd_f) * args.steps / elapsed / 1e12
    n_atomics = n_valid * 576 * ((h + 31) // 32)

    def path_record(m, atomic, ws_bytes):
        rec = {"dkv_path": "atomic" if atomic else "split", "bwd_call_ms": round(m["call"], 4),
               "preprocess_ms": round(m["pre"], 4), "postprocess_ms": round(m["post"], 4),
               "whole_backward_ms": round(m["backward"], 4),
               "whole_backward_tflops": round(bwd_f / (m["backward"] * 1e-3) / 1e12, 3),
               "frac_whole_backward": round(bwd_f / (m["backward"] * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)}
        if not atomic:
            rec["deterministic"] = True
            rec["workspace_gb"] = round(ws_bytes / 1e9, 3)
        return rec

    other = None
    if not args.no_other_path:
        m2, _, ws2 = run(not use_atomic, max(3, min(args.steps, 10)), 2)
        other = path_record(m2, not use_atomic, ws2)
    cpu = None
    if not args.no_cpu_baseline:
        from oracle import sparse_mla as sm
        qf, kvf, dof = q.cpu().double().numpy(), kv.cpu().double().numpy(), do.cpu().double().numpy()
        done, flop_done, t_cpu = 0, 0.0, 0.0
        for tok in range(t - 1, -1, -4):  # every 4th token, full lists first
            if t_cpu >= args.cpu_budget:
                break
            t1 = time.perf_counter()
            sm.sparse_mla_bwd(qf[tok:tok + 1], kvf, idx_cpu[tok:tok + 1].numpy(), dof[tok:tok + 1], scale)
            t_cpu += time.perf_counter() - t1
            nv = int((idx_cpu[tok] >= 0).sum())
            flop_done += 2.0 * nv * h * (576 + 512) * 2 + 2.0 * nv * h * (576 + 512 + 576 + 576 + 512)
            done += 1
        cpu = {"value": round(flop_done / t_cpu / 1e12, 6), "unit": "TFLOP/s", "cores": int(_blas_threads()),
               "kind": "oracle", "sample": f"{done} of {t} tokens (every 4th from the last), fwd+bwd in fp64, "
                                           f"{t_cpu:.1f} s; the same per-entry FLOP count"}
    call_tf = bwd_f / (ms["call"] * 1e-3) / 1e12
    if use_atomic:
        roof = {"kernel": "smla_bwd_kernel", "bound": "mfma", "achieved": round(call_tf, 3),
                "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": round(call_tf / PEAK_BF16_TFLOPS, 4),
                "traffic": recorded_traffic(w["name"], "bwd", SMLA_SOURCES)}
    else:
        # The deterministic call launches the sort, the backward kernel and the
        # sum together: its time (all three) prices the backward's FLOPs.
        roof = {"kernel": "attn_sparse_mla_bwd_split (sort + smla_bwd_kernel + dkv_sum)", "bound": "mfma",
                "achieved": round(call_tf, 3), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": round(call_tf / PEAK_BF16_TFLOPS, 4),
                "traffic": recorded_traffic(w["name"], "bwd_split", SMLA_SOURCES)}
    print(json.dumps({
        "metric": "sparse MLA fwd+bwd TFLOP/s (bf16)", "value": round(value, 3), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(elapsed / args.steps * 1e3, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": w["name"], "tokens": t, "kv_tokens": t, "heads": h, "topk": k,
                   "valid_entries": n_valid, "dim_qk": 576, "dim_v": 512,
                   "dkv_path": "atomic" if use_atomic else "split"},
        "fwd_kernel_ms": round(ms["fwd"], 4), "fwd_tflops": round(fwd_f / (ms["fwd"] * 1e-3) / 1e12, 3),
        "bwd_kernel_ms": round(ms["call"], 4), "bwd_tflops": round(call_tf, 3),
        **path_record(ms, use_atomic, ws),
        **({"atomics": {"count": n_atomics, "per_s": round(n_atomics / (ms["call"] * 1e-3) / 1e9, 1), "unit": "G/s"}}
           if use_atomic else {}),
        **({"other_path": other} if other else {}),
        "roofline": roof,
        **({"cpu_baseline": cpu} if cpu else {}),
    }), flush=True)


def bench_sweep(args, bd, torch):
    """Every workload, causal setting and dQ path: each call of the path timed
    on its own with HIP events (20 warm-up, 50 timed calls, medians), a 512 MB
    buffer written before each timed call so that no input is still in the
    256 MB MALL.  One JSON line per case."""
    from attention_backward_fwd_amd.synthetic import WORKLOADS, workload_inputs

    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()
    flush = torch.empty(512 << 18, dtype=torch.float32, device=dev)
    n_warm, n_time = 20, 50

    def timed(fn):
        for _ in range(n_warm):
            fn()
        ts = []
        for _ in range(n_time):
            flush.fill_(1.0)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            fn()
            e1.record(stream)
            ts.append((e0, e1))
        torch.cuda.synchronize()
        return sorted(a.elapsed_time(b) for a, b in ts)[n_time // 2]

    for w in WORKLOADS.values():
        inp = {n: t.to(dev) for n, t in workload_inputs(w).items()}
        q, k, v, do = inp["q"], inp["k"], inp["v"], inp["do"]
        sh = bd.shape_of(q, k)
        o = torch.empty_like(q)
        lse = torch.empty((w.batch, w.heads_q, w.seqlen), dtype=torch.float32, device=dev)
        nq = q.numel()
        nkv = k.numel()
        rows = w.batch * w.heads_q * w.seqlen
        for causal in w.causal:
            for path in w.paths:
                ua = path == "atomic"
                bb = bd.BwdBuffers(q, k, causal, ua)
                t_fwd = timed(lambda: bd.attn_fwd(q, k, v, o, lse, sh, w.scale, causal, stream))
                t_pre = timed(lambda: bd.attn_bwd_preprocess(o, do, bb.delta, bb.dq_accum if ua else None, sh, stream))
                t_bwd = timed(lambda: bd.attn_bwd(q, k, v, do, lse, bb.delta, bb.dq_accum, bb.dk, bb.dv, bb.workspace,
                                                  sh, w.scale, causal, ua, stream))
                t_post = timed(lambda: bd.attn_bwd_postprocess(bb.dq_accum, bb.workspace, bb.dq, bb.dk, bb.dv, sh,
                                                               stream))
                fwd_f, bwd_f = flops(w, causal)
                pre_bytes = 4 * nq + 4 * rows + (4 * nq if ua else 0)
                # grouped heads: the fp32 dK/dV partials (the atomic path's whole workspace) read, bf16 dK/dV written
                post_bytes = 6 * nq + ((bd.attn_bwd_workspace_bytes(sh, causal, 1) + 4 * nkv) if w.groups > 1 else 0)
                t_back = t_pre + t_bwd + t_post
                print(json.dumps({
                    "mode": "sweep", "workload": w.name, "causal": causal, "dq_path": path,
                    "fwd_ms": round(t_fwd, 4), "fwd_tflops": round(fwd_f / t_fwd / 1e9, 1),
                    "preprocess_ms": round(t_pre, 4), "preprocess_gbs": round(pre_bytes / t_pre / 1e6, 1),
                    "bwd_call_ms": round(t_bwd, 4), "bwd_call_tflops": round(bwd_f / t_bwd / 1e9, 1),
                    "postprocess_ms": round(t_post, 4), "postprocess_gbs": round(post_bytes / t_post / 1e6, 1),
                    "backward_ms": round(t_back, 4), "backward_tflops": round(bwd_f / t_back / 1e9, 1),
                    "backward_pct_of_peak": round(100 * bwd_f / t_back / 1e9 / PEAK_BF16_TFLOPS, 2),
                    "fwd_bwd_tflops": round((fwd_f + bwd_f) / (t_fwd + t_back) / 1e9, 1),
                    "timing": f"median of {n_time} calls after {n_warm} warm-up, HIP events, MALL flushed"}),
                    flush=True)
                del bb


def time_other_path(args, w, bd, torch, inp, o, lse, causal, use_atomic, stream):
    """The dQ path the headline did not take, on the same inputs and forward
    outputs, timed after the headline's timed region: per step preprocess ->
    attn_bwd -> postprocess (HIP events around the attn_bwd call and around
    the three), and on the split path the fixed-order sum once more on its
    own (attn_bwd_dq_sum), so that the call splits into kernel and sum."""
    q, k, v, do = inp["q"], inp["k"], inp["v"], inp["do"]
    sh = bd.shape_of(q, k)
    bb = bd.BwdBuffers(q, k, causal, use_atomic)
    n = args.steps
    ev = {m: [torch.cuda.Event(enable_timing=True) for _ in range(2 * n)] for m in ("call", "back", "sum")}

    def step(i=None):
        def rec(m, j):
            if i is not None:
                ev[m][2 * i + j].record(stream)
        rec("back", 0)
        bd.attn_bwd_preprocess(o, do, bb.delta, bb.dq_accum if use_atomic else None, sh, stream)
        rec("call", 0)
        bd.attn_bwd(q, k, v, do, lse, bb.delta, bb.dq_accum, bb.dk, bb.dv, bb.workspace, sh, w.scale, causal,
                    use_atomic, stream)
        rec("call", 1)
        bd.attn_bwd_postprocess(bb.dq_accum, bb.workspace, bb.dq, bb.dk, bb.dv, sh, stream)
        rec("back", 1)
        if not use_atomic:
            rec("sum", 0)
            bd.attn_bwd_dq_sum(bb.workspace, bb.dq_accum, sh, causal, stream)
            rec("sum", 1)

    for _ in range(args.warmup):
        step()
    for i in range(n):
        step(i)
    torch.cuda.synchronize()

    def avg(m):
        return sum(ev[m][2 * i].elapsed_time(ev[m][2 * i + 1]) for i in range(n)) / n

    _, bwd_f = flops(w, causal)
    call_ms, back_ms = avg("call"), avg("back")
    out = {"bwd_call_ms": round(call_ms, 4)}
    if use_atomic:
        kernel_ms = call_ms
    else:
        sum_ms = avg("sum")
        kernel_ms = call_ms - sum_ms
        out["sum_ms"] = round(sum_ms, 4)
        out["kernel_ms"] = round(kernel_ms, 4)
    out.update({
        "backward_ms": round(back_ms, 4),
        "backward_tflops": round(bwd_f / (back_ms * 1e-3) / 1e12, 3),
        "frac": round(bwd_f / (back_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
        "kernel_tflops": round(bwd_f / (kernel_ms * 1e-3) / 1e12, 3),
        "kernel_frac": round(bwd_f / (kernel_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
    })
    del bb
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--causal", type=int, default=None, help="override the workload's causal setting")
    ap.add_argument("--use-atomic", type=int, default=1, choices=(0, 1))
    ap.add_argument("--cpu-budget", type=float, default=12.0, help="seconds of oracle work for cpu_baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-other-path", action="store_true",
                    help="skip timing the other dQ path (split when the headline is atomic, and vice versa)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="instead of the benchmark, run a plain fp32 copy kernel over MIB MiB "
                         "(reference for scaling the HBM byte counters)")
    ap.add_argument("--merge-parts", type=int, default=0, metavar="P",
                    help="instead of the fwd+bwd step, time attn_merge of P partial (O, LSE) results "
                         "of the workload's query shape (the context-parallel merge; HBM-bound)")
    ap.add_argument("--varlen", action="store_true",
                    help="instead of the dense step, time the step over the packed causal pack of "
                         "variable-length sequences (16384 tokens, 32 heads of 128)")
    ap.add_argument("--gla", action="store_true",
                    help="instead of the attention step, time the simple gated linear attention chunk backward "
                         "(B=4, T=4096, H=32, D=128)")
    ap.add_argument("--smla", action="store_true",
                    help="instead of the attention step, time sparse MLA forward + backward "
                         "(4096 tokens, 32 heads, 2048 entries per token)")
    ap.add_argument("--sweep", action="store_true",
                    help="time fwd / preprocess / bwd / postprocess separately for every workload and dQ path")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path (attention shards over "
              "(batch, KV head) with no exchange between GPUs, so each GPU would run this same one-GPU problem)",
              file=sys.stderr)
        sys.exit(2)

    import torch

    from attention_backward_fwd_amd import binding as bd
    from attention_backward_fwd_amd.synthetic import WORKLOADS, workload_inputs

    if args.copy_calibration:
        n = args.copy_calibration * (1 << 20) // 4
        a = torch.randn(n, device="cuda:0")
        b = torch.empty_like(a)
        for _ in range(3):
            torch.mul(a, 1.0, out=b)  # one elementwise kernel: reads n*4 bytes, writes n*4 bytes
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes_read": n * 4, "bytes_written": n * 4, "launches": 3}))
        return

    if args.sweep:
        bench_sweep(args, bd, torch)
        return
    if args.varlen:
        bench_varlen(args, bd, torch)
        return
    if args.gla:
        bench_gla(args, bd, torch)
        return
    if args.smla:
        bench_smla(args, bd, torch)
        return
    w = WORKLOADS[args.workload]
    if args.merge_parts:
        bench_merge(args, w, bd, torch)
        return
    causal = w.causal[-1] if args.causal is None else bool(args.causal)
    use_atomic = args.use_atomic
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    inp = {n: t.to(dev) for n, t in workload_inputs(w).items()}
    q, k, v, do = inp["q"], inp["k"], inp["v"], inp["do"]
    sh = bd.shape_of(q, k)
    o = torch.empty_like(q)
    lse = torch.empty((w.batch, w.heads_q, w.seqlen), dtype=torch.float32, device=dev)
    bb = bd.BwdBuffers(q, k, causal, use_atomic)
    stream = torch.cuda.current_stream()

    ev = {n: [torch.cuda.Event(enable_timing=True) for _ in range(2 * args.steps)] for n in ("fwd", "bwd", "back")}

    def step(i=None):
        if i is not None:
            ev["fwd"][2 * i].record(stream)
        bd.attn_fwd(q, k, v, o, lse, sh, w.scale, causal, stream)
        if i is not None:
            ev["fwd"][2 * i + 1].record(stream)
            ev["back"][2 * i].record(stream)
        bd.attn_bwd_preprocess(o, do, bb.delta, bb.dq_accum if use_atomic else None, sh, stream)
        if i is not None:
            ev["bwd"][2 * i].record(stream)
        bd.attn_bwd(q, k, v, do, lse, bb.delta, bb.dq_accum, bb.dk, bb.dv, bb.workspace, sh, w.scale, causal,
                    use_atomic, stream)
        if i is not None:
            ev["bwd"][2 * i + 1].record(stream)
        bd.attn_bwd_postprocess(bb.dq_accum, bb.workspace, bb.dq, bb.dk, bb.dv, sh, stream)
        if i is not None:
            ev["back"][2 * i + 1].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0

    fwd_f, bwd_f = flops(w, causal)
    ms_per_step = elapsed / args.steps * 1e3
    value = (fwd_f + bwd_f) * args.steps / elapsed / 1e12
    fwd_ms = sum(ev["fwd"][2 * i].elapsed_time(ev["fwd"][2 * i + 1]) for i in range(args.steps)) / args.steps
    bwd_ms = sum(ev["bwd"][2 * i].elapsed_time(ev["bwd"][2 * i + 1]) for i in range(args.steps)) / args.steps
    back_ms = sum(ev["back"][2 * i].elapsed_time(ev["back"][2 * i + 1]) for i in range(args.steps)) / args.steps
    bwd_tflops = bwd_f / (bwd_ms * 1e-3) / 1e12
    path = "atomic" if use_atomic else "split"
    kernel = "bwd_kernel" if use_atomic else "bwd_kernel + dq_sum_kernel"

    out = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "batch": w.batch, "heads_q": w.heads_q, "heads_kv": w.heads_kv,
                   "seq_len": w.seqlen, "head_dim": w.head_dim, "causal": causal, "dq_path": path,
                   "parallelism": "none (1 GPU)"},
        "pct_of_peak": round(100.0 * value / PEAK_BF16_TFLOPS, 3),
        "fwd_kernel_ms": round(fwd_ms, 4),
        "fwd_tflops": round(fwd_f / (fwd_ms * 1e-3) / 1e12, 3),
        "bwd_kernel_ms": round(bwd_ms, 4),
        "backward_ms": round(back_ms, 4),
        "backward_tflops": round(bwd_f / (back_ms * 1e-3) / 1e12, 3),
        "roofline": {"kernel": kernel, "bound": "mfma", "achieved": round(bwd_tflops, 3), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(bwd_tflops / PEAK_BF16_TFLOPS, 4),
                     "traffic": recorded_traffic(w.name, path)},
    }
    rl = out["roofline"]
    rl["traffic_source"] = (f"recorded, not measured in this run: rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE of the "
                            f"backward kernel at sources hash {kernel_source_hash()} (profiles/traffic.json); "
                            "null when the sources changed since")
    util = recorded_util(w.name, path)
    rl["clock_adjusted_util"] = util["mfma_busy_frac"] if util else None
    rl["clock_adjusted_util_source"] = (
        f"recorded, not measured in this run: SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / 8 x 1024 SIMDs) of "
        f"the backward kernel (profiles/mfma_util.json, XCD-average clock "
        f"{util['clock_ghz'] if util else 'n/a'} GHz); null when the sources changed since")
    if not args.no_other_path:
        other = "split" if use_atomic else "atomic"
        out[other] = time_other_path(args, w, bd, torch, inp, o, lse, causal, 1 - use_atomic, stream)
    if use_atomic:
        # The atomic path's other bound: every query row receives one fp32 add
        # per element from each key block (256 keys at head_dim 128, 512 at 64) it sees.
        bn = 512 if w.head_dim == 64 else 256
        n_blk = -(-w.seqlen // bn)
        blocks_seen = sum(s // bn + 1 for s in range(w.seqlen)) if causal else w.seqlen * n_blk
        n_atomics = blocks_seen * w.batch * w.heads_q * w.head_dim
        out["dq_atomics"] = {"count": n_atomics, "per_s": round(n_atomics / (bwd_ms * 1e-3) / 1e9, 1), "unit": "G/s"}
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w, causal, args.cpu_budget)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
