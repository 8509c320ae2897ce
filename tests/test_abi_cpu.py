"""The C ABI without a GPU: the library loads, exports every function that
include/mlstm.h declares, and rejects invalid calls on the host with the
exact status before touching any device.

Pointers passed here are fake addresses: the library never dereferences a
pointer on the host, and every call below fails validation, so no HIP call is
made."""
import ctypes
import os
import re
import subprocess

import pytest

from xlstm_mlstm_matrix_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mlstm.h")

OK, NULL, SHAPE, UNSUP, STATE, WS, ALIAS = 0, 1, 2, 3, 4, 5, 6


def declared_functions():
    with open(HEADER) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mlstm_[a-z_0-9]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(B.LIB_PATH):
        from xlstm_mlstm_matrix_amd import build
        build.build()
    return B.lib()


def test_exports_every_declared_function(lib):
    names = declared_functions()
    assert len(names) == 15, names
    out = subprocess.run(["nm", "-D", "--defined-only", B.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\sT\s+(mlstm_\w+)", out))
    assert set(names) <= exported, set(names) - exported
    assert set(names) == set(B.SIGNATURES), "binding signatures out of step with the header"
    for n in names:
        getattr(lib, n)


def test_status_strings(lib):
    for s in range(11):
        assert B.status_string(s).startswith(B.STATUS[s])
    assert "unknown" in B.status_string(99)
    assert lib.mlstm_version().decode().startswith("mlstm-gfx950")


def ws(*args, variant=0):
    n = ctypes.c_size_t(12345)
    s = B.lib().mlstm_fwd_chunkwise_workspace_size_variant(*args, variant, ctypes.byref(n))
    return s, n.value


def test_workspace_query(lib):
    s, n = ws(8, 8, 4096, 256, 512, 64, B.BF16)
    assert s == OK and n > 0
    # the fused schedule keeps only a copy of n0/m0 (B*H*(d_qk+1) floats, padded)
    s, nf = ws(8, 8, 4096, 256, 512, 64, B.BF16, variant=1)
    assert s == OK and nf == (64 * 257 + 63) // 64 * 64 * 4
    # the segmented schedule holds per-segment states
    s, nseg = ws(8, 8, 4096, 256, 512, 64, B.BF16, variant=2)
    assert s == OK and nseg > nf + 64 * (256 * 512) * 4
    assert ws(0, 8, 4096, 256, 512, 64, B.BF16)[0] == SHAPE
    assert ws(1, 1, 0, 64, 64, 64, B.F32)[0] == SHAPE
    assert ws(1, 1, 64, 24, 64, 64, B.F32)[0] == UNSUP      # d_qk not a multiple of 16
    assert ws(1, 1, 64, 64, 528, 64, B.F32)[0] == UNSUP     # d_v > 512
    assert ws(1, 1, 64, 272, 64, 64, B.F32)[0] == UNSUP     # d_qk > 256
    assert ws(1, 1, 64, 64, 64, 48, B.F32)[0] == UNSUP      # chunk not supported
    assert ws(1, 1, 64, 64, 64, 64, 7)[0] == UNSUP          # dtype
    assert ws(1, 1, 64, 64, 64, 64, B.F32, variant=9)[0] == UNSUP
    assert B.lib().mlstm_fwd_chunkwise_workspace_size(1, 1, 64, 64, 64, 64, 0, None) == NULL


def sched(*args, variant=0):
    kc, ns = ctypes.c_int(-1), ctypes.c_int(-1)
    s = B.lib().mlstm_fwd_chunkwise_schedule(*args, variant, ctypes.byref(kc), ctypes.byref(ns))
    return s, kc.value, ns.value


def test_schedule_query(lib):
    # 7B-layer prefill: one workgroup per (pair, value tile) already fills the chip
    assert sched(8, 8, 4096, 256, 512, 64, B.BF16) == (OK, 64, 1)
    # long context, few pairs: segmented; chunk 128 tiles of d_qk 256 exceed LDS
    s, kc, ns = sched(1, 8, 65536, 256, 512, 128, B.BF16)
    assert (s, kc) == (OK, 64) and ns >= 2
    assert sched(1, 8, 65536, 256, 512, 128, B.BF16, variant=1) == (OK, 64, 1)
    assert sched(1, 1, 64, 16, 16, 16, B.F32, variant=1) == (OK, 16, 1)
    assert sched(1, 1, 64, 24, 16, 16, B.F32)[0] == UNSUP
    assert B.lib().mlstm_fwd_chunkwise_schedule(1, 1, 64, 16, 16, 16, 0, 0, None, None) == NULL


@pytest.mark.parametrize("io", [0, 1])
def test_every_documented_shape_is_supported(lib, io):
    """d_qk, d_v multiples of 16 up to 256 / 512 and every chunk: a schedule
    exists, with a kernel chunk that is a power of two in [16, chunk]."""
    for dk in range(16, 257, 16):
        for dv in (16, 48, 64, 80, 128, 176, 256, 320, 512):
            for chunk in (16, 32, 64, 128):
                s, kc, ns = sched(2, 2, 300, dk, dv, chunk, io)
                assert s == OK, (dk, dv, chunk)
                assert 16 <= kc <= chunk and kc & (kc - 1) == 0 and ns >= 1, (dk, dv, chunk, kc)


class Fake:
    """Fake device addresses laid out far apart (never dereferenced)."""

    def __init__(self):
        self.next = 1 << 40

    def __call__(self, nbytes):
        a = self.next
        self.next += (nbytes + (1 << 20)) // (1 << 20) * (1 << 20) + (1 << 20)
        return a


def fwd_args(B_=2, H=3, T=70, dk=64, dv=64, chunk=32, io=B.F32, state=True, out_state=True):
    fa = Fake()
    es = 2 if io == B.BF16 else 4
    P = B_ * H
    a = dict(q=fa(P * T * dk * es), k=fa(P * T * dk * es), v=fa(P * T * dv * es),
             i=fa(P * T * 4), f=fa(P * T * 4), o=fa(P * T * dv * es),
             C0=fa(P * dk * dv * 4) if state else None, n0=fa(P * dk * 4) if state else None,
             m0=fa(P * 4) if state else None, h=fa(P * T * dv * es),
             CT=fa(P * dk * dv * 4) if out_state else None, nT=fa(P * dk * 4) if out_state else None,
             mT=fa(P * 4) if out_state else None)
    s, n = ws(B_, H, T, dk, dv, chunk, io)
    assert s == OK
    a.update(ws=fa(n), wsn=n, dims=(B_, H, T, dk, dv, chunk, io))
    return a


def call_fwd(a, variant=0):
    return B.lib().mlstm_fwd_chunkwise_variant(
        a["q"], a["k"], a["v"], a["i"], a["f"], a["o"], a["C0"], a["n0"], a["m0"],
        a["h"], a["CT"], a["nT"], a["mT"], *a["dims"], variant, a["ws"], a["wsn"], None)


def test_fwd_validation(lib):
    for key in ("q", "k", "v", "i", "f", "o", "h"):
        a = fwd_args(); a[key] = None
        assert call_fwd(a) == NULL, key
    a = fwd_args(); a["dims"] = (2, 3, 0, 64, 64, 32, B.F32)
    assert call_fwd(a) == SHAPE
    a = fwd_args(); a["dims"] = (2, 3, 70, 64, 64, 24, B.F32)
    assert call_fwd(a) == UNSUP
    a = fwd_args(); a["n0"] = None
    assert call_fwd(a) == STATE
    a = fwd_args(); a["mT"] = None
    assert call_fwd(a) == STATE
    a = fwd_args(); a["ws"] = None
    assert call_fwd(a) == WS
    a = fwd_args(); a["wsn"] -= 4
    assert call_fwd(a) == WS
    # aliasing: h over an input, partial overlap of state buffers, workspace over an input
    a = fwd_args(); a["h"] = a["v"] + 64
    assert call_fwd(a) == ALIAS
    a = fwd_args(); a["CT"] = a["C0"] + 16
    assert call_fwd(a) == ALIAS
    a = fwd_args(); a["nT"] = a["C0"]
    assert call_fwd(a) == ALIAS
    a = fwd_args(); a["ws"] = a["q"]
    assert call_fwd(a) == ALIAS
    a = fwd_args(); a["h"] = a["CT"]
    assert call_fwd(a) == ALIAS


def step_args(B_=4, H=2, dk=64, dv=128, io=B.BF16, state=True):
    fa = Fake()
    es = 2 if io == B.BF16 else 4
    P = B_ * H
    a = dict(q=fa(P * dk * es), k=fa(P * dk * es), v=fa(P * dv * es), i=fa(P * 4), f=fa(P * 4),
             o=fa(P * dv * es), C=fa(P * dk * dv * 4) if state else None,
             n=fa(P * dk * 4) if state else None, m=fa(P * 4) if state else None,
             h=fa(P * dv * es), Co=fa(P * dk * dv * 4), no=fa(P * dk * 4), mo=fa(P * 4),
             dims=(B_, H, dk, dv, io))
    return a


def call_step(a):
    return B.lib().mlstm_step(a["q"], a["k"], a["v"], a["i"], a["f"], a["o"], a["C"], a["n"], a["m"],
                              a["h"], a["Co"], a["no"], a["mo"], *a["dims"], a.get("ws"),
                              a.get("wsn", 0), None)


def test_step_validation(lib):
    for key in ("q", "k", "v", "i", "f", "o", "h", "Co", "no", "mo"):
        a = step_args(); a[key] = None
        assert call_step(a) == NULL, key
    a = step_args(); a["dims"] = (0, 2, 64, 128, B.BF16)
    assert call_step(a) == SHAPE
    a = step_args(); a["dims"] = (4, 2, 40, 128, B.BF16)
    assert call_step(a) == UNSUP
    a = step_args(); a["dims"] = (4, 2, 64, 128, 5)
    assert call_step(a) == UNSUP
    a = step_args(); a["m"] = None
    assert call_step(a) == STATE
    a = step_args(); a["Co"] = a["C"] + 16
    assert call_step(a) == ALIAS
    a = step_args(); a["h"] = a["o"]
    assert call_step(a) == ALIAS
    a = step_args(); a["no"] = a["Co"] + 16
    assert call_step(a) == ALIAS


def sws(*args):
    n = ctypes.c_size_t(12345)
    s = B.lib().mlstm_step_workspace_size(*args, ctypes.byref(n))
    return s, n.value


def test_step_workspace_query(lib):
    # d_v = 512: 128 threads per row, 4 rows per pass, 16 rows per thread ->
    # blocks of 64 rows; partial read-outs [BH][blocks][d_v + 4] float32
    assert sws(256, 8, 256, 512, B.BF16) == (OK, 2048 * 4 * 516 * 4)
    assert sws(2, 3, 80, 512, B.F32) == (OK, 6 * 2 * 516 * 4)       # 64 + 16 rows
    assert sws(2, 3, 256, 256, B.F32) == (OK, 6 * 2 * 260 * 4)      # blocks of 128 rows
    assert sws(2, 3, 64, 512, B.BF16) == (OK, 0)     # one block: no split
    assert sws(2, 3, 256, 64, B.BF16) == (OK, 0)     # 32 rows per pass: one block
    assert sws(0, 3, 64, 64, B.BF16)[0] == SHAPE
    assert sws(2, 3, 40, 64, B.BF16)[0] == UNSUP
    assert sws(2, 3, 64, 64, 7)[0] == UNSUP
    assert B.lib().mlstm_step_workspace_size(1, 1, 64, 64, 0, None) == NULL


def test_step_workspace_validation(lib):
    dims = dict(B_=2, H=3, dk=256, dv=512)
    need = sws(2, 3, 256, 512, B.BF16)[1]
    free = lambda a: a["mo"] + (1 << 24)   # past every fake tensor
    a = step_args(**dims); a["ws"] = free(a); a["wsn"] = need - 4
    assert call_step(a) == WS
    a = step_args(**dims); a["ws"] = a["C"]; a["wsn"] = need
    assert call_step(a) == ALIAS
    a = step_args(**dims); a["ws"] = a["h"] - 16; a["wsn"] = need
    assert call_step(a) == ALIAS
    a = step_args(**dims); a["ws"] = free(a) + 8; a["wsn"] = need
    assert call_step(a) == 8   # MLSTM_ERR_ALIGN


def call_step_noalloc(a):
    return B.lib().mlstm_step_noalloc(a["q"], a["k"], a["v"], a["i"], a["f"], a["o"], a["C"], a["n"],
                                      a["m"], a["h"], a["Co"], a["no"], a["mo"], *a["dims"], None)


def test_step_noalloc_validation(lib):
    # the checks of mlstm_step, then the scratch limit, all before any HIP call
    for key in ("q", "k", "v", "i", "f", "o", "h", "Co", "no", "mo"):
        a = step_args(); a[key] = None
        assert call_step_noalloc(a) == NULL, key
    a = step_args(); a["dims"] = (0, 2, 64, 128, B.BF16)
    assert call_step_noalloc(a) == SHAPE
    a = step_args(); a["dims"] = (4, 2, 40, 128, B.BF16)
    assert call_step_noalloc(a) == UNSUP
    a = step_args(); a["n"] = None
    assert call_step_noalloc(a) == STATE
    a = step_args(); a["h"] = a["o"]
    assert call_step_noalloc(a) == ALIAS
    a = step_args(); a["q"] += 4
    assert call_step_noalloc(a) == 8   # MLSTM_ERR_ALIGN
    # the partials of 4064 cells of 256 x 512 fit in the 32 MiB scratch; of 4065 they do not
    assert sws(4064, 1, 256, 512, B.BF16)[1] <= B.STEP_NOALLOC_MAX_BYTES < sws(4065, 1, 256, 512, B.BF16)[1]
    a = step_args(B_=4065, H=1, dk=256, dv=512)
    assert call_step_noalloc(a) == 10  # MLSTM_ERR_SCRATCH
    a = step_args(B_=1000, H=5, dk=256, dv=512, state=False)
    assert call_step_noalloc(a) == 10
    assert "mlstm_step_noalloc" in B.status_string(10)


def test_binding_refuses_cpu_tensors():
    import torch
    x = torch.zeros(1, 1, 4, 16)
    with pytest.raises(Exception):
        B.fwd_chunkwise(x, x, x, torch.zeros(1, 1, 4), torch.zeros(1, 1, 4), x)


# ---- backward: host-side validation only (every call below returns before any
# device work; the fake addresses are never dereferenced)

def bws(*args):
    n = ctypes.c_size_t(12345)
    s = B.lib().mlstm_bwd_chunkwise_workspace_size(*args, ctypes.byref(n))
    return s, n.value


def test_bwd_workspace_query(lib):
    # per pair and chunk: the state record (C', n', m; padded to 4 floats),
    # the rows a [32][dv], P and P~ [2][32][32], four scalars per token, the
    # carried-gradient record (G*, g*; padded); then the chunk totals
    # (padded), 64 dm0 partials and the checkpoint pass's K, V tiles
    up4 = lambda x: (x + 3) // 4 * 4
    for dk, dv in ((64, 48), (128, 64)):
        s, n = bws(2, 3, 70, dk, dv, 32, B.F32)
        nch, rec, grec = 3, up4(dk * dv + dk + 1), up4(dk * dv + dk)
        per_pair = nch * (rec + 32 * dv + 2 * 32 * 32 + 4 * 32 + grec) + up4(nch) + 64 + 32 * (dk + dv)
        assert s == OK and n == 6 * per_pair * 4, (dk, dv)
    assert bws(2, 3, 70, 256, 512, 32, B.BF16)[0] == OK
    assert bws(2, 3, 70, 272, 64, 32, B.F32)[0] == UNSUP     # d_qk above 256
    assert bws(2, 3, 70, 64, 528, 32, B.BF16)[0] == UNSUP    # d_v above 512
    assert bws(2, 3, 70, 24, 64, 32, B.F32)[0] == UNSUP      # not a multiple of 16
    assert bws(1, 1, (1 << 20) - 64, 256, 512, 32, B.BF16)[0] == OK
    assert bws(1, 1, (1 << 20) - 32, 256, 512, 32, B.BF16)[0] == UNSUP   # (T + 32) * 512 floats = 2 GiB
    assert bws(2, 3, 70, 64, 64, 48, B.F32)[0] == UNSUP      # chunk
    assert bws(2, 3, 0, 64, 64, 32, B.F32)[0] == SHAPE
    assert bws(2, 3, 70, 64, 64, 32, 5)[0] == UNSUP          # dtype
    assert B.lib().mlstm_bwd_chunkwise_workspace_size(1, 1, 64, 64, 64, 32, 0, None) == NULL


def bwd_call(a, **over):
    x = dict(a)
    x.update(over)
    B_, H, T, dk, dv, chunk, io = x["dims"]
    return B.lib().mlstm_bwd_chunkwise(
        x["q"], x["k"], x["v"], x["i"], x["f"], x["o"], x["C0"], x["n0"], x["m0"], x["dh"],
        x["gq"], x["gk"], x["gv"], x["gi"], x["gf"], x["go"], x["gC0"], x["gn0"], x["gm0"],
        B_, H, T, dk, dv, chunk, io, x["ws"], x["wsn"], None)


def bwd_args(B_=2, H=3, T=70, dk=64, dv=48, io=B.F32):
    fa = Fake()
    es = 2 if io == B.BF16 else 4
    P = B_ * H
    a = dict(q=fa(P * T * dk * es), k=fa(P * T * dk * es), v=fa(P * T * dv * es),
             i=fa(P * T * 4), f=fa(P * T * 4), o=fa(P * T * dv * es),
             C0=fa(P * dk * dv * 4), n0=fa(P * dk * 4), m0=fa(P * 4), dh=fa(P * T * dv * es),
             gq=fa(P * T * dk * 4), gk=fa(P * T * dk * 4), gv=fa(P * T * dv * 4), gi=fa(P * T * 4),
             gf=fa(P * T * 4), go=fa(P * T * dv * 4), gC0=fa(P * dk * dv * 4), gn0=fa(P * dk * 4),
             gm0=fa(P * 4))
    s, n = bws(B_, H, T, dk, dv, 32, io)
    assert s == OK
    a.update(ws=fa(n), wsn=n, dims=(B_, H, T, dk, dv, 32, io))
    return a


def test_bwd_validation(lib):
    a = bwd_args()
    assert bwd_call(a, gq=None) == NULL
    assert bwd_call(a, dh=None) == NULL
    assert bwd_call(a, n0=None) == STATE
    assert bwd_call(a, gm0=None) == STATE
    assert bwd_call(a, wsn=a["wsn"] - 4) == WS
    assert bwd_call(a, ws=None) == WS
    assert bwd_call(a, gq=a["q"]) == ALIAS                      # output over an input
    assert bwd_call(a, gk=a["gq"] + 64) == ALIAS                # two outputs overlap
    assert bwd_call(a, gC0=a["ws"]) == ALIAS                    # output over the workspace
    assert bwd_call(a, dims=(2, 3, 70, 272, 48, 32, B.F32)) == UNSUP
    assert bwd_call(a, dims=(2, 3, 0, 64, 48, 32, B.F32)) == SHAPE


def test_misaligned_pointers_rejected(lib):
    """Every entry point rejects a pointer off a 16-byte boundary before any
    device work (fake addresses, never dereferenced)."""
    ALIGN = 8
    for key in ("q", "k", "v", "i", "f", "o", "C0", "n0", "m0", "h", "CT", "nT", "mT", "ws"):
        a = fwd_args(); a[key] += 4
        assert call_fwd(a) == ALIGN, key
    for key in ("q", "v", "i", "C", "h", "Co", "mo"):
        a = step_args(); a[key] += 2
        assert call_step(a) == ALIGN, key
    b = bwd_args()
    for key in ("q", "dh", "gq", "gf", "gC0", "ws"):
        assert bwd_call(b, **{key: b[key] + 2}) == ALIGN, key


# ---- layer: host-side validation only (every call below returns before any
# device work; the fake addresses are never dereferenced)

def lws(*args):
    n = ctypes.c_size_t(12345)
    s = B.lib().mlstm_layer_fwd_workspace_size(*args, ctypes.byref(n))
    return s, n.value


def test_layer_workspace_query(lib):
    # B=2 T=70 d_model=64 H=3 d_qk=16 d_v=32 chunk 32 float32: 32 MiB for the
    # GEMMs, then q, k, v, o~, i~, f~ of the 3*2 cells (each padded to 256
    # bytes), W_i and W_f stacked [2H, d_model] (one gate GEMM), then the
    # cell's own workspace
    s, n = lws(2, 70, 64, 3, 16, 32, 32, B.F32)
    cell = ctypes.c_size_t(0)
    assert B.lib().mlstm_fwd_chunkwise_workspace_size(3, 2, 70, 16, 32, 32, B.F32, ctypes.byref(cell)) == OK
    up = lambda x: (x + 255) // 256 * 256
    HBT = 3 * 2 * 70
    assert s == OK
    assert n == ((32 << 20) + 2 * up(HBT * 16 * 4) + 2 * up(HBT * 32 * 4) + 2 * up(HBT * 4)
                 + up(2 * 3 * 64 * 4) + up(cell.value))
    assert lws(2, 70, 60, 3, 16, 32, 32, B.F32)[0] == UNSUP    # d_model not a multiple of 8
    assert lws(2, 70, 64, 3, 24, 32, 32, B.F32)[0] == UNSUP    # d_qk
    assert lws(2, 70, 64, 3, 16, 32, 48, B.F32)[0] == UNSUP    # chunk
    assert lws(0, 70, 64, 3, 16, 32, 32, B.F32)[0] == SHAPE
    assert lws(2, 70, 64, 3, 16, 32, 32, 4)[0] == UNSUP        # dtype
    assert B.lib().mlstm_layer_fwd_workspace_size(1, 1, 8, 1, 16, 16, 16, 0, None) == NULL


def layer_args(B_=2, T=70, D=64, H=3, dk=16, dv=32, io=B.BF16):
    fa = Fake()
    es = 2 if io == B.BF16 else 4
    a = dict(x=fa(B_ * T * D * es), Wq=fa(H * dk * D * es), Wk=fa(H * dk * D * es),
             Wv=fa(H * dv * D * es), Wo=fa(H * dv * D * es), Wi=fa(H * D * es), Wf=fa(H * D * es),
             bq=fa(H * dk * 4), bk=fa(H * dk * 4), bv=fa(H * dv * 4), bo=fa(H * dv * 4), bi=fa(H * 4),
             bf=fa(H * 4), C0=None, n0=None, m0=None, h=fa(H * B_ * T * dv * es),
             CT=None, nT=None, mT=None, dims=(B_, T, D, H, dk, dv, 32, io))
    a["wsn"] = lws(*a["dims"])[1]
    a["ws"] = fa(a["wsn"])
    return a


def call_layer(a):
    k = ("x", "Wq", "Wk", "Wv", "Wo", "Wi", "Wf", "bq", "bk", "bv", "bo", "bi", "bf", "C0", "n0", "m0",
         "h", "CT", "nT", "mT")
    return B.lib().mlstm_layer_fwd(*(a[x] for x in k), *a["dims"], a["ws"], a["wsn"], None)


def test_layer_validation(lib):
    for key in ("x", "Wq", "Wk", "Wv", "Wo", "Wi", "Wf", "bq", "bk", "bv", "bo", "bi", "bf", "h"):
        a = layer_args(); a[key] = None
        assert call_layer(a) == NULL, key
    a = layer_args(); a["dims"] = (2, 70, 60, 3, 16, 32, 32, B.BF16)
    assert call_layer(a) == UNSUP
    a = layer_args(); a["wsn"] -= 16
    assert call_layer(a) == WS
    a = layer_args(); a["ws"] = None
    assert call_layer(a) == WS
    a = layer_args(); a["Wq"] += 8
    assert call_layer(a) == 8   # MLSTM_ERR_ALIGN
    a = layer_args(); a["h"] = a["x"]
    assert call_layer(a) == ALIAS
    a = layer_args(); a["ws"] = a["Wv"]
    assert call_layer(a) == ALIAS


def with_layer_state(a, inplace=False):
    fa = Fake()
    fa.next = 1 << 44  # far from the addresses layer_args handed out
    B_, T, D, H, dk, dv = a["dims"][:6]
    P = H * B_
    a.update(C0=fa(P * dk * dv * 4), n0=fa(P * dk * 4), m0=fa(P * 4))
    if inplace:
        a.update(CT=a["C0"], nT=a["n0"], mT=a["m0"])
    else:
        a.update(CT=fa(P * dk * dv * 4), nT=fa(P * dk * 4), mT=fa(P * 4))
    return a


def test_layer_validation_precedes_device_work(lib):
    # The cell's own checks (state triples, alignment of the state and h,
    # overlap of h / the final state / the workspace) run before the first
    # projection is enqueued: each of these returns its validation status, not
    # MLSTM_ERR_HIP from a device call.
    for key in ("C0", "n0", "m0", "CT", "nT", "mT"):
        a = with_layer_state(layer_args()); a[key] = None
        assert call_layer(a) == STATE, key
    for key in ("C0", "n0", "m0", "h", "CT", "nT", "mT"):
        a = with_layer_state(layer_args()); a[key] += 4
        assert call_layer(a) == 8, key   # MLSTM_ERR_ALIGN
    a = layer_args(); a["h"] = a["ws"] + 256       # h inside the workspace
    assert call_layer(a) == ALIAS
    a = with_layer_state(layer_args()); a["CT"] = a["ws"]
    assert call_layer(a) == ALIAS
    a = with_layer_state(layer_args()); a["nT"] = a["h"]
    assert call_layer(a) == ALIAS
    a = with_layer_state(layer_args()); a["C0"] = a["ws"] + 1024   # read state inside the workspace
    assert call_layer(a) == ALIAS
    a = with_layer_state(layer_args()); a["h"] = a["C0"]
    assert call_layer(a) == ALIAS
    a = with_layer_state(layer_args()); a["CT"] = a["C0"] + 16     # partial overlap, not in place
    assert call_layer(a) == ALIAS
    a = with_layer_state(layer_args()); a["nT"] = a["C0"]          # another state buffer
    assert call_layer(a) == ALIAS
    # in place but with h overlapping the state: still rejected (an exact
    # in-place call with valid buffers would reach device work, which these
    # fake addresses must never do)
    a = with_layer_state(layer_args(), inplace=True); a["h"] = a["m0"]
    assert call_layer(a) == ALIAS


# ---- sLSTM: host-side validation only

def slstm_args(B_=2, H=3, T=50, d=32, io=B.BF16, state=True):
    fa = Fake()
    es = 2 if io == B.BF16 else 4
    ns = B_ * H * d * 4
    a = dict(gx=fa(B_ * H * T * 4 * d * es), R=fa(H * 4 * d * d * es),
             c0=fa(ns) if state else None, n0=fa(ns) if state else None,
             m0=fa(ns) if state else None, h0=fa(ns) if state else None,
             h=fa(B_ * H * T * d * es), cT=fa(ns), nT=fa(ns), mT=fa(ns), hT=fa(ns),
             dims=(B_, H, T, d, io))
    return a


def call_slstm(a):
    k = ("gx", "R", "c0", "n0", "m0", "h0", "h", "cT", "nT", "mT", "hT")
    return B.lib().mlstm_slstm_fwd(*(a[x] for x in k), *a["dims"], None)


def test_slstm_validation(lib):
    for key in ("gx", "R", "h"):
        a = slstm_args(); a[key] = None
        assert call_slstm(a) == NULL, key
    for dims, st in (((2, 3, 50, 24, B.BF16), UNSUP), ((2, 3, 50, 144, B.BF16), UNSUP),
                     ((2, 3, 0, 32, B.BF16), SHAPE), ((2, 3, 50, 32, 3), UNSUP)):
        a = slstm_args(); a["dims"] = dims
        assert call_slstm(a) == st, dims
    a = slstm_args(); a["m0"] = None
    assert call_slstm(a) == STATE
    a = slstm_args(); a["hT"] = None
    assert call_slstm(a) == STATE
    a = slstm_args(); a["R"] += 8
    assert call_slstm(a) == 8   # MLSTM_ERR_ALIGN
    a = slstm_args(); a["h"] = a["gx"]
    assert call_slstm(a) == ALIAS
    a = slstm_args(); a["cT"] = a["n0"]
    assert call_slstm(a) == ALIAS
    a = slstm_args(); a["cT"] = a["c0"] + 16
    assert call_slstm(a) == ALIAS
