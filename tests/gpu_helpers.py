"""Shared helpers of the GPU tests: run the HIP path through the C ABI."""

import math
import sys

import numpy as np
import torch

from attention_backward_fwd_amd import binding as bd

TOL = 2e-2  # max|gpu - oracle| <= TOL * max|oracle|, per tensor


def gqa_parts(b, s, hq, g, d):
    """dK/dV partials per (key row, KV head) of the backward's workspace, by
    the rule the header states: the smallest divisor P of the group size with
    b * Hkv * P * key blocks >= 512, else the group size."""
    blocks = b * (hq // g) * math.ceil(s / (512 if d == 64 else 256))
    return next((p for p in range(1, g) if g % p == 0 and blocks * p >= 512), g)


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def to_dev(inp, device="cuda"):
    return {n: t.to(device) for n, t in inp.items()}


def run_path(d, causal, scale, use_atomic, poison=True):
    """fwd -> preprocess -> bwd (-> sum) -> postprocess on device tensors.

    Every output and scratch buffer starts as NaN when ``poison`` is set, so
    an element the kernels fail to write shows up as NaN.
    """
    q, k, v, do = d["q"], d["k"], d["v"], d["do"]
    sh = bd.shape_of(q, k)
    nan = float("nan")
    o = torch.full_like(q, nan) if poison else torch.empty_like(q)
    lse = torch.full((q.shape[0], q.shape[2], q.shape[1]), nan, dtype=torch.float32, device=q.device)
    bd.attn_fwd(q, k, v, o, lse, sh, scale, causal)
    bb = bd.BwdBuffers(q, k, causal, use_atomic)
    if poison:
        for t in (bb.delta, bb.dq_accum, bb.dq, bb.dk, bb.dv) + ((bb.workspace,) if bb.workspace is not None else ()):
            t.fill_(nan)
    bd.attn_bwd_preprocess(o, do, bb.delta, bb.dq_accum if use_atomic else None, sh)
    bd.attn_bwd(q, k, v, do, lse, bb.delta, bb.dq_accum, bb.dk, bb.dv, bb.workspace, sh, scale, causal, use_atomic)
    bd.attn_bwd_postprocess(bb.dq_accum, bb.workspace, bb.dq, bb.dk, bb.dv, sh)
    torch.cuda.synchronize()
    return {"o": o, "lse": lse, "delta": bb.delta, "dq": bb.dq, "dk": bb.dk, "dv": bb.dv, "dq_accum": bb.dq_accum}


def np64(t):
    return t.detach().to("cpu", torch.float64).numpy()


def err_ratio(gpu, ref, zero_scale=None):
    """max|gpu - ref| / max|ref|.

    Where the exact result is identically zero (e.g. dQ and dK at S = 1), the
    kernel's value is pure rounding noise and the relative measure is
    undefined; the error is then taken relative to ``zero_scale`` (the
    magnitude of the problem's other gradients) and must stay far below it.
    """
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if not np.all(np.isfinite(gpu)):
        return float("inf")
    scale = np.max(np.abs(ref)) if ref.size else 0.0
    if scale == 0.0:
        if zero_scale is None or zero_scale == 0.0:
            return 0.0 if np.max(np.abs(gpu), initial=0.0) == 0.0 else float("inf")
        return float(np.max(np.abs(gpu), initial=0.0) / zero_scale) * 100.0
    return float(np.max(np.abs(gpu - ref)) / scale)
