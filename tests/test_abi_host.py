"""Host-side tests of the C ABI (no GPU needed).

Every call here fails an argument check, which the library performs on the
host before any HIP call, so nothing is launched.  Fake device addresses are
never dereferenced.
"""

import ctypes
import math

import pytest

from attention_backward_fwd_amd import binding as bd
from tests.gpu_helpers import gqa_parts

P = ctypes.c_void_p
A = P(0x10000)      # 16-byte aligned fake device address
MIS = P(0x10008)    # misaligned


def lib():
    return bd.library()


def shp(b=2, s=300, hq=8, g=2, d=128):
    return bd.attn_shape(b, s, hq, g, d)


def test_library_exports_every_header_symbol():
    names = bd.header_functions()
    assert names == sorted(["attn_fwd", "attn_bwd_preprocess", "attn_bwd_workspace_bytes", "attn_bwd",
                            "attn_bwd_postprocess", "attn_bwd_dq_sum", "attn_bwd_noalloc", "attn_merge", "attn_strerror", "attn_fwd_varlen",
                            "attn_bwd_varlen_workspace_bytes", "attn_bwd_varlen",
                            "attn_bwd_varlen_postprocess", "gla_chunk_bwd_workspace_bytes", "gla_chunk_bwd",
                            "attn_sparse_mla_fwd", "attn_sparse_mla_bwd_preprocess", "attn_sparse_mla_bwd",
                            "attn_sparse_mla_bwd_postprocess", "attn_sparse_mla_bwd_split_workspace_bytes",
                            "attn_sparse_mla_bwd_split"])
    for n in names:
        assert hasattr(lib(), n), n


def test_every_kernel_launch_stub_is_defined():
    """A kernel whose host launch stub the compiler dropped leaves the symbol
    undefined; the library then loads lazily on the host but fails on the GPU
    when the loader resolves it."""
    import shutil
    import subprocess
    nm = shutil.which("nm")
    if nm is None:
        pytest.skip("nm not available")
    und = subprocess.run([nm, "-u", bd.LIB_PATH], capture_output=True, text=True, check=True).stdout
    assert "__device_stub__" not in und
    defined = subprocess.run([nm, "--defined-only", bd.LIB_PATH], capture_output=True, text=True, check=True).stdout
    for kernel in ("fwd_kernel", "bwd_kernel", "dq_sum_kernel", "preprocess_kernel", "postprocess_kernel"):
        assert f"__device_stub__{kernel}" in defined, kernel


def test_strerror_covers_every_code():
    msgs = {lib().attn_strerror(c).decode() for c in range(0, -10, -1)}
    assert len(msgs) == 10
    assert lib().attn_strerror(-99).decode() == "unknown status"


@pytest.mark.parametrize("g", [1, 4])
@pytest.mark.parametrize("s", [1, 128, 256, 257, 4096])
def test_workspace_bytes(g, s):
    sh = shp(b=2, s=s, hq=8, g=g, d=64)
    nq = 2 * s * 8 * 64
    nblk = math.ceil(s / 512)  # key blocks of 512 at head_dim 64
    gqa = 2 * nq * 4 if g > 1 else 0
    for causal in (0, 1):
        assert lib().attn_bwd_workspace_bytes(sh, causal, 1) == gqa
        assert lib().attn_bwd_workspace_bytes(sh, causal, 0) == gqa + nblk * nq * 4


@pytest.mark.parametrize("b,s,hq,g,d,parts", [
    (8, 2048, 32, 4, 128, 1),   # 8*8*8 = 512 workgroups with one partial per KV head
    (1, 8192, 64, 8, 128, 2),   # 8*32 = 256: two partials of four heads each
    (2, 1024, 48, 4, 64, 4),    # 2*12*2 = 48: one partial per query head
    (6, 300, 96, 6, 128, 3),    # 6*16*2 = 192: P = 2 gives 384, P = 3 gives 576
    (4, 300, 96, 6, 128, 6),    # 4*16*2 = 128: 1, 2, 3 give 128, 256, 384 -> the group size
])
def test_workspace_bytes_gqa_partials(b, s, hq, g, d, parts):
    assert gqa_parts(b, s, hq, g, d) == parts
    nkv = b * s * (hq // g) * d
    nblk = math.ceil(s / (512 if d == 64 else 256))
    sh = shp(b=b, s=s, hq=hq, g=g, d=d)
    assert lib().attn_bwd_workspace_bytes(sh, 1, 1) == 2 * nkv * parts * 4
    assert lib().attn_bwd_workspace_bytes(sh, 0, 0) == 2 * nkv * parts * 4 + nblk * b * s * hq * d * 4


def test_workspace_bytes_follow_the_stated_partial_rule():
    """attn_bwd_workspace_bytes against the rule the header states, over a
    spread of grouped shapes (grids on both sides of 512 workgroups)."""
    n = 0
    for b in (1, 2, 3, 8, 22, 64):
        for hq, g in ((8, 2), (16, 4), (24, 3), (32, 8), (48, 6), (64, 8), (96, 16)):
            for s in (1, 255, 256, 513, 2048):
                for d in (64, 128):
                    if b * s * hq * d >= (1 << 31):
                        continue
                    sh = shp(b=b, s=s, hq=hq, g=g, d=d)
                    nkv = b * s * (hq // g) * d
                    nblk = math.ceil(s / (512 if d == 64 else 256))
                    gqa = 2 * nkv * gqa_parts(b, s, hq, g, d) * 4
                    assert lib().attn_bwd_workspace_bytes(sh, 1, 1) == gqa, (b, hq, g, s, d)
                    assert lib().attn_bwd_workspace_bytes(sh, 1, 0) == gqa + nblk * b * s * hq * d * 4
                    n += 1
    assert n > 300


def test_workspace_bytes_block_height_follows_head_dim():
    # 256-key blocks at head_dim 128: S = 300 needs 2 slots, S = 256 one.
    for s_, nblk in ((256, 1), (257, 2), (300, 2), (4096, 16)):
        nq = 2 * s_ * 8 * 128
        assert lib().attn_bwd_workspace_bytes(shp(b=2, s=s_, hq=8, g=1, d=128), 1, 0) == nblk * nq * 4


def test_workspace_bytes_invalid_is_zero():
    assert lib().attn_bwd_workspace_bytes(shp(hq=6, g=4), 0, 0) == 0
    assert lib().attn_bwd_workspace_bytes(shp(d=96), 0, 0) == 0
    assert lib().attn_bwd_workspace_bytes(shp(), 2, 0) == 0


def fwd(**kw):
    args = dict(q=A, k=A, v=A, o=A, lse=A, shape=shp(), scale=0.1, causal=1, stream=None)
    args.update(kw)
    return lib().attn_fwd(args["q"], args["k"], args["v"], args["o"], args["lse"], args["shape"],
                          args["scale"], args["causal"], args["stream"])


def pre(**kw):
    args = dict(o=A, do=A, delta=A, dq=A, shape=shp(), stream=None)
    args.update(kw)
    return lib().attn_bwd_preprocess(args["o"], args["do"], args["delta"], args["dq"], args["shape"], args["stream"])


def bwd(**kw):
    args = dict(q=A, k=A, v=A, do=A, lse=A, delta=A, dq=A, dk=A, dv=A, ws=A, wsb=1 << 40, shape=shp(), scale=0.1,
                causal=1, atomic=1, stream=None)
    args.update(kw)
    return lib().attn_bwd(args["q"], args["k"], args["v"], args["do"], args["lse"], args["delta"], args["dq"],
                          args["dk"], args["dv"], args["ws"], args["wsb"], args["shape"], args["scale"],
                          args["causal"], args["atomic"], args["stream"])


def post(**kw):
    args = dict(dq_accum=A, ws=A, wsb=1 << 40, dq=A, dk=A, dv=A, shape=shp(), stream=None)
    args.update(kw)
    return lib().attn_bwd_postprocess(args["dq_accum"], args["ws"], args["wsb"], args["dq"], args["dk"], args["dv"],
                                      args["shape"], args["stream"])


def noalloc(**kw):
    args = dict(q=A, k=A, v=A, do=A, lse=A, delta=A, dq=A, dk=A, dv=A, shape=shp(), scale=0.1, causal=1,
                stream=None)
    args.update(kw)
    return lib().attn_bwd_noalloc(args["q"], args["k"], args["v"], args["do"], args["lse"], args["delta"],
                                  args["dq"], args["dk"], args["dv"], args["shape"], args["scale"], args["causal"],
                                  args["stream"])


E = {"null": -1, "shape": -2, "hd": -3, "align": -4, "range": -5, "ws": -6, "flag": -8, "scratch": -9}


@pytest.mark.parametrize("kw,code", [
    ({"q": None}, "null"), ({"lse": None}, "null"),
    ({"shape": shp(b=0)}, "shape"), ({"shape": shp(s=0)}, "shape"), ({"shape": shp(hq=6, g=4)}, "shape"),
    ({"shape": shp(g=0)}, "shape"), ({"shape": shp(d=96)}, "hd"), ({"shape": shp(d=256)}, "hd"),
    ({"shape": shp(b=64, s=8192, hq=64, g=1, d=128)}, "range"),
    ({"shape": shp(b=1, s=2, hq=65536, g=1, d=128)}, "range"),
    ({"scale": 0.0}, "range"), ({"scale": -1.0}, "range"), ({"scale": float("nan")}, "range"),
    ({"scale": float("inf")}, "range"), ({"causal": 2}, "flag"), ({"o": MIS}, "align"), ({"lse": MIS}, "align"),
])
def test_fwd_errors(kw, code):
    assert fwd(**kw) == E[code]


@pytest.mark.parametrize("kw,code", [
    ({"o": None}, "null"), ({"delta": None}, "null"), ({"shape": shp(hq=7, g=2)}, "shape"),
    ({"shape": shp(d=32)}, "hd"), ({"dq": MIS}, "align"), ({"do": MIS}, "align"),
])
def test_preprocess_errors(kw, code):
    assert pre(**kw) == E[code]


@pytest.mark.parametrize("kw,code", [
    ({"dq": None}, "null"), ({"lse": None}, "null"),
    ({"shape": shp(g=1), "dk": None}, "null"),
    ({"shape": shp(hq=0)}, "shape"), ({"shape": shp(d=80)}, "hd"),
    ({"atomic": 3}, "flag"), ({"causal": -1}, "flag"),
    ({"scale": float("-inf")}, "range"),
    ({"ws": None}, "ws"), ({"wsb": 1024}, "ws"),
    ({"atomic": 0, "shape": shp(g=1), "ws": None}, "ws"),
    ({"delta": MIS}, "align"), ({"ws": MIS}, "align"),
])
def test_bwd_errors(kw, code):
    assert bwd(**kw) == E[code]


@pytest.mark.parametrize("kw,code", [
    ({"dq": None}, "null"), ({"dk": None}, "null"), ({"ws": None}, "ws"), ({"wsb": 16}, "ws"),
    ({"shape": shp(s=-3)}, "shape"), ({"dq_accum": MIS}, "align"),
])
def test_postprocess_errors(kw, code):
    assert post(**kw) == E[code]


def merge(**kw):
    args = dict(op=A, lp=A, n=3, o=A, lse=A, shape=shp(), stream=None)
    args.update(kw)
    return lib().attn_merge(args["op"], args["lp"], args["n"], args["o"], args["lse"], args["shape"], args["stream"])


@pytest.mark.parametrize("kw,code", [
    ({"op": None}, "null"), ({"lse": None}, "null"), ({"n": 0}, "shape"), ({"n": -2}, "shape"),
    ({"shape": shp(s=0)}, "shape"), ({"shape": shp(d=96)}, "hd"), ({"shape": shp(b=64, s=8192, hq=64, g=1)}, "range"),
    ({"o": MIS}, "align"), ({"lp": MIS}, "align"),
])
def test_merge_errors(kw, code):
    assert merge(**kw) == E[code]


def test_python_shape_helpers():
    import torch
    q = torch.empty((2, 17, 8, 64))
    k = torch.empty((2, 17, 2, 64))
    sh = bd.shape_of(q, k)
    assert (sh.batch, sh.seqlen, sh.heads_q, sh.groups, sh.head_dim) == (2, 17, 8, 4, 64)
    with pytest.raises(ValueError):
        bd.shape_of(q, torch.empty((2, 17, 3, 64)))


# ------------------------------------------------------------ packed sequences

def vshp(n=3, t=1000, m=400, hq=8, g=2, d=128, tk=None, mk=None):
    return bd.attn_varlen_shape(n, t, t if tk is None else tk, m, m if mk is None else mk, hq, g, d)


@pytest.mark.parametrize("g", [1, 4])
@pytest.mark.parametrize("mk", [0, 1, 256, 257, 4096])
def test_varlen_workspace_bytes(g, mk):
    sh = vshp(n=5, t=3000, m=700, hq=8, g=g, d=64, tk=2000, mk=mk)
    nq, nk = 3000 * 8 * 64, 2000 * 8 * 64
    gqa = 2 * nk * 4 if g > 1 else 0
    for causal in (0, 1):
        assert lib().attn_bwd_varlen_workspace_bytes(sh, causal, 1) == gqa
        assert lib().attn_bwd_varlen_workspace_bytes(sh, causal, 0) == gqa + math.ceil(mk / 512) * nq * 4
    assert lib().attn_bwd_varlen_workspace_bytes(vshp(hq=6, g=4), 0, 0) == 0
    assert lib().attn_bwd_varlen_workspace_bytes(vshp(), 0, 7) == 0


def vfwd(**kw):
    args = dict(q=A, k=A, v=A, o=A, lse=A, cu=A, cuk=A, shape=vshp(), scale=0.1, causal=1, stream=None)
    args.update(kw)
    return lib().attn_fwd_varlen(args["q"], args["k"], args["v"], args["o"], args["lse"], args["cu"], args["cuk"],
                                 args["shape"], args["scale"], args["causal"], args["stream"])


def vbwd(**kw):
    args = dict(q=A, k=A, v=A, do=A, lse=A, delta=A, dq=A, dk=A, dv=A, ws=A, wsb=1 << 40, cu=A, cuk=A,
                shape=vshp(), scale=0.1, causal=1, atomic=1, stream=None)
    args.update(kw)
    return lib().attn_bwd_varlen(args["q"], args["k"], args["v"], args["do"], args["lse"], args["delta"],
                                 args["dq"], args["dk"], args["dv"], args["ws"], args["wsb"], args["cu"],
                                 args["cuk"], args["shape"], args["scale"], args["causal"], args["atomic"],
                                 args["stream"])


def vpost(**kw):
    args = dict(dq_accum=A, ws=A, wsb=1 << 40, dq=A, dk=A, dv=A, shape=vshp(), stream=None)
    args.update(kw)
    return lib().attn_bwd_varlen_postprocess(args["dq_accum"], args["ws"], args["wsb"], args["dq"], args["dk"],
                                             args["dv"], args["shape"], args["stream"])


@pytest.mark.parametrize("kw,code", [
    ({"q": None}, "null"), ({"cu": None}, "null"), ({"cuk": None}, "null"), ({"lse": None}, "null"),
    ({"k": None}, "null"),
    ({"shape": vshp(n=-1)}, "shape"), ({"shape": vshp(t=-1)}, "shape"), ({"shape": vshp(m=-1)}, "shape"),
    ({"shape": vshp(tk=-5)}, "shape"), ({"shape": vshp(mk=-5)}, "shape"),
    ({"shape": vshp(hq=0)}, "shape"), ({"shape": vshp(hq=6, g=4)}, "shape"), ({"shape": vshp(d=96)}, "hd"),
    ({"shape": vshp(t=1 << 20, hq=64, g=1)}, "range"), ({"shape": vshp(tk=1 << 20, hq=64, g=1)}, "range"),
    ({"shape": vshp(hq=65536, g=1)}, "range"),
    ({"shape": vshp(n=1 << 20, m=1 << 16, hq=64, g=1, t=1000)}, "range"),
    ({"scale": 0.0}, "range"), ({"causal": 3}, "flag"), ({"o": MIS}, "align"), ({"v": MIS}, "align"),
])
def test_fwd_varlen_errors(kw, code):
    assert vfwd(**kw) == E[code]


@pytest.mark.parametrize("kw,code", [
    ({"dq": None}, "null"), ({"cu": None}, "null"), ({"cuk": None}, "null"), ({"v": None}, "null"),
    ({"shape": vshp(g=1), "dv": None}, "null"),
    ({"shape": vshp(hq=7, g=2)}, "shape"), ({"shape": vshp(d=32)}, "hd"),
    ({"atomic": 2}, "flag"), ({"scale": float("nan")}, "range"),
    ({"ws": None}, "ws"), ({"wsb": 64}, "ws"), ({"atomic": 0, "shape": vshp(g=1), "ws": None}, "ws"),
    ({"delta": MIS}, "align"), ({"ws": MIS}, "align"),
])
def test_bwd_varlen_errors(kw, code):
    assert vbwd(**kw) == E[code]


@pytest.mark.parametrize("kw,code", [
    ({"dq": None}, "null"), ({"dk": None}, "null"), ({"ws": None}, "ws"), ({"wsb": 16}, "ws"),
    ({"shape": vshp(t=-3)}, "shape"), ({"dq_accum": MIS}, "align"),
])
def test_varlen_postprocess_errors(kw, code):
    assert vpost(**kw) == E[code]


def test_varlen_empty_pack_is_a_no_op():
    """No rows: every check still runs, then nothing is enqueued (NULL
    pointers allowed), so this runs without a GPU."""
    empty = vshp(n=2, t=0, m=5, tk=0)
    assert vfwd(q=None, k=None, v=None, o=None, lse=None, cu=None, cuk=None, shape=empty) == 0
    assert vfwd(q=None, k=None, v=None, o=None, lse=None, cu=None, cuk=None, shape=vshp(t=0, tk=50)) == 0
    assert vbwd(q=None, k=None, v=None, do=None, lse=None, delta=None, dq=None, dk=None, dv=None, ws=None,
                cu=None, cuk=None, shape=empty) == 0
    assert vpost(dq_accum=None, ws=None, dq=None, dk=None, dv=None, shape=vshp(t=0, tk=0)) == 0
    assert vpost(dq_accum=None, ws=None, dq=None, dk=None, dv=None, shape=vshp(t=0, tk=9, g=1)) == 0
    assert vfwd(q=None, shape=empty, causal=2) == E["flag"]
    assert vbwd(q=None, shape=bd.attn_varlen_shape(2, 0, 0, 5, 5, 8, 2, 96)) == E["hd"]


def test_varlen_shape_helper():
    import torch
    q = torch.empty((50, 8, 64))
    k = torch.empty((70, 2, 64))
    sh = bd.varlen_shape_of(q, k, 4, 20, 30)
    assert (sh.n_seqs, sh.total_q, sh.total_k, sh.max_seqlen_q, sh.max_seqlen_k, sh.heads_q, sh.groups,
            sh.head_dim) == (4, 50, 70, 20, 30, 8, 4, 64)
    assert bd.varlen_shape_of(q, k, 4, 20).max_seqlen_k == 20


# ------------------------------------------------------------ simple GLA

def gshp(b=2, t=300, h=4, d=128):
    return bd.gla_shape(b, t, h, d)


@pytest.mark.parametrize("t", [1, 64, 65, 4096])
def test_gla_workspace_bytes(t):
    # per-token q.dq and k.dk: [2][B*H][T] fp32
    want = 2 * (2 * 4) * t * 4
    assert lib().gla_chunk_bwd_workspace_bytes(gshp(t=t)) == want
    assert lib().gla_chunk_bwd_workspace_bytes(gshp(d=64)) == 0
    assert lib().gla_chunk_bwd_workspace_bytes(gshp(b=0)) == 0


def gbwd(**kw):
    args = dict(q=A, k=A, v=A, g=A, do=A, dq=A, dk=A, dv=A, dg=A, ws=A, wsb=1 << 40, shape=gshp(), scale=0.1,
                stream=None)
    args.update(kw)
    return lib().gla_chunk_bwd(args["q"], args["k"], args["v"], args["g"], args["do"], args["dq"], args["dk"],
                               args["dv"], args["dg"], args["ws"], args["wsb"], args["shape"], args["scale"],
                               args["stream"])


@pytest.mark.parametrize("kw,code", [
    ({"q": None}, "null"), ({"g": None}, "null"), ({"dg": None}, "null"),
    ({"shape": gshp(b=0)}, "shape"), ({"shape": gshp(t=0)}, "shape"), ({"shape": gshp(h=0)}, "shape"),
    ({"shape": gshp(d=64)}, "hd"), ({"shape": gshp(b=64, t=8192, h=64)}, "range"),
    ({"shape": gshp(b=300, t=4, h=300)}, "range"),
    ({"scale": 0.0}, "range"), ({"scale": float("nan")}, "range"),
    ({"ws": None}, "ws"), ({"wsb": 100}, "ws"),
    ({"q": MIS}, "align"), ({"ws": MIS}, "align"), ({"g": P(0x10002)}, "align"),
])
def test_gla_errors(kw, code):
    assert gbwd(**kw) == E[code]


def test_gla_g_needs_only_4_byte_alignment():
    """g and dg are fp32 per-token values: 4-byte aligned is enough (the call
    then fails only on the workspace, which the test leaves too small)."""
    assert gbwd(g=P(0x10004), dg=P(0x10004), wsb=8) == E["ws"]


# ------------------------------------------------------------ sparse MLA

def mshp(t=8, tk=100, h=16, k=64, dqk=576, dv=512):
    return bd.smla_shape(t, tk, h, k, dqk, dv)


def mfwd(**kw):
    args = dict(q=A, kv=A, idx=A, o=A, lse=A, shape=mshp(), scale=0.05, stream=None)
    args.update(kw)
    return lib().attn_sparse_mla_fwd(args["q"], args["kv"], args["idx"], args["o"], args["lse"], args["shape"],
                                     args["scale"], args["stream"])


@pytest.mark.parametrize("kw,code", [
    ({"q": None}, "null"), ({"idx": None}, "null"), ({"lse": None}, "null"),
    ({"shape": mshp(t=0)}, "shape"), ({"shape": mshp(tk=0)}, "shape"), ({"shape": mshp(h=0)}, "shape"),
    ({"shape": mshp(k=0)}, "shape"), ({"shape": mshp(dqk=512)}, "hd"), ({"shape": mshp(dv=576)}, "hd"),
    ({"shape": mshp(k=8193)}, "range"), ({"shape": mshp(t=1 << 20, h=64)}, "range"),
    ({"shape": mshp(tk=(1 << 19) + 1)}, "range"),
    ({"scale": 0.0}, "range"), ({"q": MIS}, "align"), ({"o": MIS}, "align"), ({"idx": P(0x10002)}, "align"),
])
def test_sparse_mla_fwd_errors(kw, code):
    assert mfwd(**kw) == E[code]


def mbwd(**kw):
    args = dict(q=A, kv=A, do=A, idx=A, lse=A, delta=A, dq=A, acc=A, shape=mshp(), scale=0.05, stream=None)
    args.update(kw)
    return lib().attn_sparse_mla_bwd(args["q"], args["kv"], args["do"], args["idx"], args["lse"], args["delta"],
                                     args["dq"], args["acc"], args["shape"], args["scale"], args["stream"])


@pytest.mark.parametrize("kw,code", [
    ({"acc": None}, "null"), ({"delta": None}, "null"), ({"shape": mshp(k=0)}, "shape"),
    ({"shape": mshp(dqk=128)}, "hd"), ({"scale": float("inf")}, "range"), ({"dq": MIS}, "align"),
    ({"acc": MIS}, "align"), ({"delta": P(0x10001)}, "align"), ({"shape": mshp(tk=(1 << 19) + 1)}, "range"),
])
def test_sparse_mla_bwd_errors(kw, code):
    assert mbwd(**kw) == E[code]


def test_sparse_mla_pre_post_errors():
    f = lib().attn_sparse_mla_bwd_preprocess
    assert f(None, A, A, None, mshp(), None) == E["null"]
    assert f(A, A, A, MIS, mshp(), None) == E["align"]
    assert f(A, A, A, None, mshp(h=0), None) == E["shape"]
    g = lib().attn_sparse_mla_bwd_postprocess
    assert g(None, A, mshp(), None) == E["null"]
    assert g(A, MIS, mshp(), None) == E["align"]


def _a256(x):
    return (x + 255) // 256 * 256


def smla_split_ws(t, tk, h, k):
    """Workspace of the deterministic sparse MLA backward, region by region:
    one fp32 row of 576 per entry slot and 32-head tile plus a sink row;
    entry positions; key-row offsets (tk + 1); two (key, entry) buffer pairs
    of the radix sort; the digit counts of its widest pass (passes of at most
    10 bits over keys 0 .. tk, tiles of 4096 entries); one scan partial per
    4096 counts."""
    n, n_ht = t * k, -(-h // 32)
    bits = tk.bit_length()
    passes = 1 if bits <= 10 else 2
    hist = (1 << -(-bits // passes)) * -(-n // 4096)
    return (_a256((n * n_ht + 1) * 2304) + _a256(4 * n) + _a256(4 * (tk + 1)) + 4 * _a256(4 * n) + _a256(4 * hist)
            + _a256(4 * -(-hist // 4096)))


@pytest.mark.parametrize("t,tk,h,k", [(8, 100, 16, 64), (8, 100, 40, 64), (3, 1023, 1, 1), (5, 1024, 33, 9),
                                      (4096, 4096, 32, 2048), (7, (1 << 19), 128, 8192)])
def test_sparse_mla_split_workspace_bytes(t, tk, h, k):
    assert bd.attn_sparse_mla_bwd_split_workspace_bytes(mshp(t=t, tk=tk, h=h, k=k)) == smla_split_ws(t, tk, h, k)


def test_sparse_mla_split_workspace_bytes_small_case_by_hand():
    # T8 K64 H16 Tk100: 513 rows * 2304 B + 2048 + 512 + 4 * 2048 + 512 (128 digits) + 256.
    assert bd.attn_sparse_mla_bwd_split_workspace_bytes(mshp()) == 1193472
    assert bd.attn_sparse_mla_bwd_split_workspace_bytes(mshp(h=0)) == 0
    assert bd.attn_sparse_mla_bwd_split_workspace_bytes(mshp(dqk=128)) == 0


def msplit(**kw):
    need = bd.attn_sparse_mla_bwd_split_workspace_bytes(mshp())
    args = dict(q=A, kv=A, do=A, idx=A, lse=A, delta=A, dq=A, dkv=A, ws=A, wsb=need, shape=mshp(), scale=0.05,
                stream=None)
    args.update(kw)
    return lib().attn_sparse_mla_bwd_split(args["q"], args["kv"], args["do"], args["idx"], args["lse"],
                                           args["delta"], args["dq"], args["dkv"], args["ws"], args["wsb"],
                                           args["shape"], args["scale"], args["stream"])


@pytest.mark.parametrize("kw,code", [
    ({"dkv": None}, "null"), ({"idx": None}, "null"), ({"shape": mshp(k=0)}, "shape"),
    ({"shape": mshp(dv=256)}, "hd"), ({"scale": float("nan")}, "range"), ({"shape": mshp(k=8193)}, "range"),
    ({"ws": None}, "ws"), ({"wsb": 1193471}, "ws"), ({"dkv": MIS}, "align"), ({"ws": MIS}, "align"),
    ({"lse": P(0x10002)}, "align"),
])
def test_sparse_mla_split_errors(kw, code):
    assert msplit(**kw) == E[code]


# Scratch of attn_bwd_noalloc: 64 MiB; need = (2P/groups if groups > 1) * nq * 4 + ceil(S/bn) * nq * 4, with
# key blocks of bn = 256 keys at head_dim 128 and 512 at head_dim 64 (P = groups at these sizes).
@pytest.mark.parametrize("kw,code", [
    ({"dk": None, "shape": shp(g=1)}, "null"), ({"dv": None}, "null"), ({"delta": None}, "null"),
    ({"shape": shp(hq=6, g=4)}, "shape"), ({"shape": shp(d=96)}, "hd"), ({"causal": 2}, "flag"),
    ({"scale": 0.0}, "range"),
    # B1 S4096 Hq8 D128, MHA: 16 blocks * 4 Mi floats * 4 B = 256 MiB.
    ({"shape": shp(b=1, s=4096, hq=8, g=1, d=128)}, "scratch"),
    # B2 S1024 Hq16 D64, GQA: (2 + 2) * 2 Mi floats * 4 B = 32 MiB fits; Hq48 (96 MiB) does not.
    ({"shape": shp(b=2, s=1024, hq=48, g=4, d=64)}, "scratch"),
    ({"shape": shp(b=2, s=1024, hq=16, g=4, d=64), "dq": MIS}, "align"),
    ({"q": MIS}, "align"),
])
def test_noalloc_errors(kw, code):
    assert noalloc(**kw) == E[code]


def dqsum(**kw):
    args = dict(ws=A, wsb=1 << 40, dq=A, shape=shp(), causal=1, stream=None)
    args.update(kw)
    return lib().attn_bwd_dq_sum(args["ws"], args["wsb"], args["dq"], args["shape"], args["causal"], args["stream"])


@pytest.mark.parametrize("kw,code", [
    ({"ws": None}, "null"), ({"dq": None}, "null"), ({"shape": shp(hq=6, g=4)}, "shape"),
    ({"shape": shp(d=32)}, "hd"), ({"causal": 3}, "flag"),
    # B2 S300 Hq8 D128, GQA-2: (2 + 2 blocks) x 614400 floats x 4 B is one byte more than given.
    ({"wsb": 4 * 614400 * 4 - 1}, "ws"),
    ({"ws": MIS}, "align"), ({"dq": MIS}, "align"),
])
def test_dq_sum_errors(kw, code):
    assert dqsum(**kw) == E[code]
