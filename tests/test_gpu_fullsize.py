"""Full-size workloads on the GPU, checked against the oracle on samples and
on whole slices.

At these sizes the oracle computes selected outputs one at a time: O, LSE,
Delta and dQ of sampled query rows (each needs only its own softmax row) and
dK, dV of sampled key rows of one KV group (each needs every query row of the
group that sees the key).  Properties that hold at any size are checked on
whole tensors: sum over keys of dK is zero (adding a constant vector to every
key leaves the output unchanged) and sum over keys of dV equals the sum of
the group's dO rows (softmax rows sum to one).

The slice test compares, element by element, every row of O, LSE and dQ of
the query heads of one KV group of one batch entry, and every key of that
group's dK and dV, with the oracle run on that batch entry and group alone.
"""

import numpy as np
import pytest
import torch

from attention_backward_fwd_amd.synthetic import WORKLOADS, workload_inputs
from oracle import attention as orc
from tests.gpu_helpers import TOL, err_ratio, np64, run_path, say, to_dev

pytestmark = pytest.mark.gpu

FULL = [
    ("mha_causal_b8_h32_s1024_d64", True, 1),
    ("mha_causal_b8_h32_s1024_d64", True, 0),
    ("gqa4_causal_b8_h32_s2048_d128", True, 1),
    ("gqa4_causal_b8_h32_s2048_d128", True, 0),
    ("mha_causal_b4_h32_s4096_d128", True, 1),
    ("mha_causal_b4_h32_s4096_d128", True, 0),
    ("gqa8_b1_h64_s8192_d128", False, 1),
    ("gqa8_b1_h64_s8192_d128", False, 0),
    ("gqa8_b1_h64_s8192_d128", True, 1),
    ("gqa8_b1_h64_s8192_d128", True, 0),
]


def _rows(S, rng):
    fixed = [0, 1, 63, 64, 127, 128, S // 2 + 3, S - 65, S - 2, S - 1]
    return sorted(set(int(x) for x in fixed + list(rng.integers(0, S, 6)) if 0 <= x < S))


@pytest.mark.parametrize("name,causal,use_atomic", FULL)
def test_full_size_sampled(name, causal, use_atomic):
    w = WORKLOADS[name]
    say(f"[full] {name} causal={causal} atomic={use_atomic}: inputs")
    inp = workload_inputs(w)
    f64 = {n: t.to(torch.float64).numpy() for n, t in inp.items()}
    dev = to_dev(inp)
    gpu = run_path(dev, causal, w.scale, use_atomic)
    say(f"[full] {name}: gpu done")
    rng = np.random.default_rng(0)
    S, B, Hq, G = w.seqlen, w.batch, w.heads_q, w.groups
    heads = sorted({(0, 0), (B - 1, Hq - 1), (int(rng.integers(0, B)), int(rng.integers(0, Hq)))})
    worst = {}
    for b, h in heads:
        rows = _rows(S, rng)
        ref = orc.attention_rows(f64["q"], f64["k"], f64["v"], f64["do"], w.scale, causal, G, b, h, rows)
        got = {"o": np64(gpu["o"][b, rows, h]), "lse": np64(gpu["lse"][b, h, rows]),
               "delta": np64(gpu["delta"][b, h, rows]), "dq": np64(gpu["dq"][b, rows, h])}
        for n in got:
            worst[n] = max(worst.get(n, 0.0), err_ratio(got[n], ref[n]))
    # dK/dV at sampled keys of one KV group
    b, kv = B - 1, (Hq // G) - 1
    cols = sorted({0, 1, 127, 128, S // 3, S - 129, S - 1})
    refc = orc.attention_cols(f64["q"], f64["k"], f64["v"], f64["do"], w.scale, causal, G, b, kv, cols)
    worst["dk"] = err_ratio(np64(gpu["dk"][b, cols, kv]), refc["dk"])
    worst["dv"] = err_ratio(np64(gpu["dv"][b, cols, kv]), refc["dv"])
    say(f"[full] {name} causal={causal} atomic={use_atomic}: " + " ".join(f"{k}={v:.2e}" for k, v in worst.items()))
    for n in ("o", "lse", "dq", "dk", "dv"):
        assert worst[n] <= TOL, (n, worst[n])

    # whole-tensor properties (fp64 sums on the device)
    dk = gpu["dk"].double()
    dv = gpu["dv"].double()
    dk_sum = dk.sum(dim=1).abs().max().item()
    dk_scale = dk.abs().sum(dim=1).max().item()
    do_grp = dev["do"].double().view(B, S, Hq // G, G, w.head_dim).sum(dim=(1, 3))
    dv_err = (dv.sum(dim=1) - do_grp).abs().max().item()
    dv_scale = dv.abs().sum(dim=1).max().item()
    say(f"[full] {name}: sum_s dK / sum_s |dK| = {dk_sum / dk_scale:.2e}; dV-sum err = {dv_err / dv_scale:.2e}")
    assert dk_sum <= 2e-2 * dk_scale
    assert dv_err <= 2e-2 * dv_scale
    for n in ("o", "lse", "dq", "dk", "dv"):
        assert torch.isfinite(gpu[n].float()).all(), n


SLICES = [(name, use_atomic) for name in ("mha_causal_b8_h32_s1024_d64", "gqa4_causal_b8_h32_s2048_d128",
                                         "mha_causal_b4_h32_s4096_d128") for use_atomic in (1, 0)]


@pytest.mark.parametrize("name,use_atomic", SLICES)
def test_full_size_whole_group_slice(name, use_atomic):
    w = WORKLOADS[name]
    causal = True
    B, S, Hq, G = w.batch, w.seqlen, w.heads_q, w.groups
    b, kv = B - 1, Hq // G - 1
    say(f"[slice] {name} atomic={use_atomic}: batch {b}, KV head {kv}")
    inp = workload_inputs(w)
    dev = to_dev(inp)
    gpu = run_path(dev, causal, w.scale, use_atomic)
    sl = {n: t[b:b + 1].to(torch.float64).numpy() for n, t in inp.items()}
    ref = orc.attention_bwd(sl["q"], sl["k"], sl["v"], sl["do"], w.scale, causal, G, heads=[kv])
    hs = list(range(kv * G, kv * G + G))
    zs = float(np.max(np.abs(ref["dv"][0, :, kv])))
    got = {"o": np64(gpu["o"][b][:, hs]), "lse": np64(gpu["lse"][b][hs]), "delta": np64(gpu["delta"][b][hs]),
           "dq": np64(gpu["dq"][b][:, hs]), "dk": np64(gpu["dk"][b][:, kv]), "dv": np64(gpu["dv"][b][:, kv])}
    want = {"o": ref["o"][0][:, hs], "lse": ref["lse"][0][hs], "delta": ref["delta"][0][hs],
            "dq": ref["dq"][0][:, hs], "dk": ref["dk"][0][:, kv], "dv": ref["dv"][0][:, kv]}
    ratios = {n: err_ratio(got[n], want[n], zero_scale=zs) for n in got}
    say(f"[slice] {name} atomic={use_atomic}: " + " ".join(f"{n}={r:.2e}" for n, r in ratios.items()))
    for n in ("o", "lse", "dq", "dk", "dv"):
        assert ratios[n] <= TOL, (n, ratios[n])


# MHA; grouped heads with one dK/dV partial per KV head (GQA-4: each backward
# workgroup sweeps the group's four query heads) and with two (GQA-8).
@pytest.mark.parametrize("name,causal", [("mha_causal_b4_h32_s4096_d128", True),
                                         ("gqa4_causal_b8_h32_s2048_d128", True),
                                         ("gqa8_b1_h64_s8192_d128", True)])
def test_split_bitwise_deterministic_full_size(name, causal):
    w = WORKLOADS[name]
    dev = to_dev(workload_inputs(w))
    a = run_path(dev, causal, w.scale, 0, poison=False)
    a = {n: a[n].clone() for n in ("dq", "dk", "dv", "dq_accum")}
    b = run_path(dev, causal, w.scale, 0, poison=True)
    for n in a:
        va = a[n].view(torch.int16) if a[n].dtype == torch.bfloat16 else a[n].view(torch.int32)
        vb = b[n].view(torch.int16) if b[n].dtype == torch.bfloat16 else b[n].view(torch.int32)
        assert torch.equal(va, vb), (name, n)
    say(f"[full] split path bitwise identical across runs: {name}")
