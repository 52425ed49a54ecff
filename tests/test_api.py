"""The C ABI on the CPU: the library loads, exports every function gdr.h
declares, and validates arguments on the host (no kernel is launched)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gdr.h")


@pytest.fixture(scope="module")
def gdr():
    import gated_delta_rule_16_amd as g
    return g


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\**\s*([a-z_0-9]+)\s*\(",
                      src, flags=re.M)


def test_header_declares_the_three_operations():
    names = declared_functions()
    for n in ("gdr_chunk_fwd", "gdr_recurrent_step", "gdr2_chunk_fwd",
              "gdr_chunk_fwd_ex", "gdr_recurrent_step_ex", "gdr2_chunk_fwd_ex",
              "gdr_output_gate", "gdr_chunk_bwd", "gdr_chunk_bwd_workspace_size",
              "gdr2_chunk_bwd", "gdr2_chunk_bwd_workspace_size",
              "gdr_chunk_fwd_split", "gdr_chunk_fwd_split_workspace_size",
              "gdr_chunk_bwd_ex", "gdr2_chunk_bwd_ex",
              "gdr_output_gate_bwd", "gdr_output_gate_bwd_workspace_size",
              "gdr_chunk_bwd_split", "gdr_chunk_bwd_split_workspace_size",
              "gdr2_chunk_fwd_split", "gdr2_chunk_bwd_split",
              "gdr2_chunk_bwd_split_workspace_size",
              "gdr_status_string", "gdr_version"):
        assert n in names, names


def test_every_declared_symbol_is_exported(gdr):
    for n in declared_functions():
        assert hasattr(gdr.lib, n), f"{n} not exported by libgdr.so"


def test_status_strings(gdr):
    assert gdr.status_string(0) == "ok"
    for c in (1, 2, 3):
        assert gdr.status_string(c) != "unknown status"
    assert gdr.lib.gdr_version() >= 200


A16 = 1 << 20          # a fake, 16-byte aligned "device" address
BAD = A16 + 4          # misaligned


def chunk(gdr, B=1, T=8, H=1, Dk=64, Dv=64, dt=1, q=A16, k=A16, v=A16,
          a=A16, b=A16, s0=None, odt=1, o=A16, sf=None):
    return gdr.lib.gdr_chunk_fwd(B, T, H, Dk, Dv, dt, q, k, v, a, b, s0, odt,
                                 o, sf, None)


def chunk2(gdr, B=1, T=8, H=1, Dk=64, Dv=64, dt=1, q=A16, k=A16, v=A16,
           a=A16, e=A16, w=A16, s0=None, odt=1, o=A16, sf=None):
    return gdr.lib.gdr2_chunk_fwd(B, T, H, Dk, Dv, dt, q, k, v, a, e, w, s0,
                                  odt, o, sf, None)


def step(gdr, N=2, H=1, Dk=64, Dv=64, dt=1, q=A16, k=A16, v=A16, a=A16,
         b=A16, s=A16, odt=1, o=A16):
    return gdr.lib.gdr_recurrent_step(N, H, Dk, Dv, dt, q, k, v, a, b, s, odt,
                                      o, None)


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), 1), (dict(k=None), 1), (dict(v=None), 1),
    (dict(a=None), 1), (dict(b=None), 1), (dict(o=None), 1),
    (dict(q=BAD), 1), (dict(v=BAD), 1), (dict(o=BAD + 1), 1),
    (dict(a=BAD + 1), 1), (dict(s0=BAD), 1), (dict(sf=BAD), 1),
    (dict(B=-1), 1), (dict(T=-1), 1), (dict(H=-1), 1),
    (dict(Dk=96), 2), (dict(Dv=32), 2), (dict(Dk=0), 2), (dict(dt=7), 2),
    (dict(odt=5), 2),
])
def test_chunk_fwd_validation(gdr, kw, code):
    assert chunk(gdr, **kw) == code


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), 1), (dict(a=None), 1), (dict(e=None), 1), (dict(w=None), 1),
    (dict(e=BAD), 1), (dict(B=-3), 1), (dict(Dk=48), 2), (dict(dt=9), 2),
])
def test_gdr2_chunk_fwd_validation(gdr, kw, code):
    assert chunk2(gdr, **kw) == code


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), 1), (dict(s=None), 1), (dict(s=BAD), 1), (dict(o=None), 1),
    (dict(N=-1), 1), (dict(Dk=256), 2), (dict(Dv=100), 2), (dict(dt=3), 2),
])
def test_recurrent_step_validation(gdr, kw, code):
    assert step(gdr, **kw) == code


def test_scalar_gates_need_element_alignment_only(gdr):
    # a T-slice of the fp32 gates is 4-byte aligned: accepted by validation
    # (checked with a size that makes the call return before any launch)
    assert chunk(gdr, a=BAD, b=BAD, Dk=96) == 2


def test_empty_calls_launch_nothing(gdr):
    # nothing to do: returns OK without touching the device
    assert chunk(gdr, B=0, q=None, k=None, v=None, a=None, b=None, o=None) == 0
    assert chunk(gdr, H=0, q=None, k=None, v=None, a=None, b=None, o=None) == 0
    assert chunk(gdr, T=0, q=None, k=None, v=None, a=None, b=None, o=None) == 0
    assert step(gdr, N=0, q=None, k=None, v=None, a=None, b=None, s=None,
                o=None) == 0
    assert chunk2(gdr, B=0, q=None) == 0


def test_binding_rejects_cpu_tensors(gdr):
    import torch
    x = torch.zeros(1, 4, 1, 64)
    with pytest.raises(ValueError):
        gdr.gdr_chunk_fwd(x, x, x, torch.zeros(1, 4, 1), torch.zeros(1, 4, 1))


def test_ex_variants_check_flags(gdr):
    """Unknown flag bits are rejected before anything else is looked at; the
    known bit goes through the same argument checks as the plain call."""
    L = gdr.lib
    for bad in (2, 4, 0x80000000, 0xffffffff):
        assert L.gdr_chunk_fwd_ex(1, 8, 1, 64, 64, 1, A16, A16, A16, A16, A16, None, 1,
                                  A16, None, bad, None) == 2
        assert L.gdr2_chunk_fwd_ex(1, 8, 1, 64, 64, 1, A16, A16, A16, A16, A16, A16, None,
                                   1, A16, None, bad, None) == 2
        assert L.gdr_recurrent_step_ex(2, 1, 64, 64, 1, A16, A16, A16, A16, A16, A16, 1,
                                       A16, bad, None) == 2
    f = gdr.GDR_L2NORM_QK
    # validation failures (no launch): NULL q, misaligned v, bad head dim
    assert L.gdr_chunk_fwd_ex(1, 8, 1, 64, 64, 1, None, A16, A16, A16, A16, None, 1,
                              A16, None, f, None) == 1
    assert L.gdr2_chunk_fwd_ex(1, 8, 1, 64, 64, 1, A16, A16, BAD, A16, A16, A16, None,
                               1, A16, None, f, None) == 1
    assert L.gdr_recurrent_step_ex(2, 1, 96, 64, 1, A16, A16, A16, A16, A16, A16, 1,
                                   A16, f, None) == 2
    # empty calls return OK with the flag set
    assert L.gdr_chunk_fwd_ex(0, 8, 1, 64, 64, 1, None, None, None, None, None, None, 1,
                              None, None, f, None) == 0
    assert L.gdr_recurrent_step_ex(0, 1, 64, 64, 1, None, None, None, None, None, None,
                                   1, None, f, None) == 0


def gate(gdr, N=4, H=2, Dv=128, odt_in=1, o=A16, gdt=1, g=A16, w=None, eps=1e-6, odt=1, y=A16):
    return gdr.lib.gdr_output_gate(N, H, Dv, odt_in, o, gdt, g, w, eps, odt, y, None)


@pytest.mark.parametrize("kw,code", [
    (dict(o=None), 1), (dict(g=None), 1), (dict(y=None), 1), (dict(o=BAD), 1),
    (dict(g=BAD), 1), (dict(y=BAD), 1), (dict(w=BAD), 1), (dict(N=-1), 1), (dict(H=-1), 1),
    (dict(eps=-1.0), 1), (dict(eps=float("nan")), 1), (dict(eps=float("inf")), 1),
    (dict(Dv=96), 2), (dict(Dv=32), 2), (dict(odt_in=3), 2), (dict(gdt=9), 2), (dict(odt=4), 2),
])
def test_output_gate_validation(gdr, kw, code):
    assert gate(gdr, **kw) == code


def test_output_gate_empty(gdr):
    assert gate(gdr, N=0, o=None, g=None, y=None) == 0
    assert gate(gdr, H=0, o=None, g=None, y=None) == 0


def bwd(gdr, B=1, T=8, H=1, Dk=64, Dv=64, dt=1, q=A16, k=A16, v=A16, a=A16, b=A16, s0=None,
        ddt=1, do=A16, dsf=None, dq=A16, dk=A16, dv=A16, da=A16, db=A16, ds0=None, ws=A16,
        wsb=None):
    if wsb is None:
        wsb = gdr.gdr_chunk_bwd_workspace_size(B, T, H, Dk, Dv)
    return gdr.lib.gdr_chunk_bwd(B, T, H, Dk, Dv, dt, q, k, v, a, b, s0, ddt, do, dsf, dq, dk, dv,
                                 da, db, ds0, ws, wsb, None)


def test_bwd_workspace_size(gdr):
    """Chunk-start states (B H ceil(T/16) Dv Dk floats), each chunk's T and
    decayed Gram (2 x 16 x 16 floats), dq and dk accumulators for the fused
    norm (2 Dk floats per token-head) and, for Dv/32 row blocks, dbeta and
    d log alpha partials (2 floats per token-head each)."""
    assert gdr.gdr_chunk_bwd_workspace_size(2, 100, 3, 128, 64) == \
        4 * (2 * 3 * 7 * 64 * 128 + 2 * 3 * 7 * 512 + 2 * 600 * 128 + 2 * 2 * 600)
    assert gdr.gdr_chunk_bwd_workspace_size(1, 8, 1, 96, 64) == 0
    assert gdr.gdr_chunk_bwd_workspace_size(-1, 8, 1, 64, 64) == 0


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), 1), (dict(do=None), 1), (dict(dq=None), 1), (dict(dv=None), 1),
    (dict(da=None), 1), (dict(ws=None), 1), (dict(ws=BAD), 1), (dict(dk=BAD), 1),
    (dict(s0=BAD), 1), (dict(dsf=BAD), 1), (dict(ds0=BAD), 1), (dict(wsb=100), 1),
    (dict(T=-1), 1), (dict(Dk=96), 2), (dict(ddt=5), 2), (dict(dt=9), 2),
])
def test_bwd_validation(gdr, kw, code):
    assert bwd(gdr, **kw) == code


def test_bwd_empty(gdr):
    assert bwd(gdr, B=0, q=None, k=None, v=None, a=None, b=None, do=None, dq=None, dk=None,
               dv=None, da=None, db=None, ws=None, wsb=0) == 0


def bwd2(gdr, B=1, T=8, H=1, Dk=64, Dv=64, dt=1, q=A16, k=A16, v=A16, a=A16, e=A16, w=A16,
         s0=None, ddt=1, do=A16, dsf=None, dq=A16, dk=A16, dv=A16, da=A16, de=A16, dw=A16,
         ds0=None, ws=A16, wsb=None):
    if wsb is None:
        wsb = gdr.gdr2_chunk_bwd_workspace_size(B, T, H, Dk, Dv)
    return gdr.lib.gdr2_chunk_bwd(B, T, H, Dk, Dv, dt, q, k, v, a, e, w, s0, ddt, do, dsf, dq, dk,
                                  dv, da, de, dw, ds0, ws, wsb, None)


def test_bwd2_workspace_size(gdr):
    """Chunk-start states (B H ceil(T/16) Dv Dk floats), each chunk's T
    (16 x 16 floats) and accumulators of dq, dk, derase and d log alpha
    (4 Dk floats per token-head)."""
    assert gdr.gdr2_chunk_bwd_workspace_size(2, 100, 3, 128, 64) == \
        4 * (2 * 3 * 7 * 64 * 128 + 2 * 3 * 7 * 256 + 4 * 600 * 128)
    assert gdr.gdr2_chunk_bwd_workspace_size(1, 8, 1, 64, 96) == 0
    assert gdr.gdr2_chunk_bwd_workspace_size(1, -8, 1, 64, 64) == 0


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), 1), (dict(a=None), 1), (dict(e=None), 1), (dict(w=BAD), 1),
    (dict(do=None), 1), (dict(dq=None), 1), (dict(da=BAD), 1), (dict(de=None), 1),
    (dict(dw=None), 1), (dict(ws=None), 1), (dict(ws=BAD), 1), (dict(s0=BAD), 1),
    (dict(dsf=BAD), 1), (dict(ds0=BAD), 1), (dict(wsb=100), 1), (dict(H=-1), 1),
    (dict(Dk=32), 2), (dict(ddt=5), 2), (dict(dt=9), 2),
])
def test_bwd2_validation(gdr, kw, code):
    assert bwd2(gdr, **kw) == code


def test_bwd2_empty(gdr):
    assert bwd2(gdr, H=0, q=None, k=None, v=None, a=None, e=None, w=None, do=None, dq=None,
                dk=None, dv=None, da=None, de=None, dw=None, ws=None, wsb=0) == 0


def split(gdr, B=1, T=64, H=1, Dk=64, Dv=64, dt=1, q=A16, k=A16, v=A16, a=A16, b=A16, s0=None,
          odt=1, o=A16, sf=None, nseg=4, flags=0, ws=A16, wsb=None):
    if wsb is None:
        wsb = gdr.lib.gdr_chunk_fwd_split_workspace_size(B, T, H, Dk, Dv, dt, nseg)
    return gdr.lib.gdr_chunk_fwd_split(B, T, H, Dk, Dv, dt, q, k, v, a, b, s0, odt, o, sf, nseg,
                                       flags, ws, wsb, None)


def test_split_workspace_size(gdr):
    """R, P and start states (fp32, 256-byte rounded), the zero v of the P pass
    (fp32 inputs only: the bf16 kernels take a missing v as zero), and the P
    pass's output (bf16) only when Dk != Dv."""
    up = lambda x: (x + 255) // 256 * 256
    f = gdr.lib.gdr_chunk_fwd_split_workspace_size
    bn = 2 * 4 * 3
    assert f(2, 96, 3, 128, 128, 1, 4) == up(bn * 128 * 128 * 4) * 3
    assert f(2, 96, 3, 128, 64, 0, 4) == (up(bn * 64 * 128 * 4) * 2 + up(bn * 128 * 128 * 4) +
                                          up(2 * 96 * 3 * 128 * 4) + up(2 * 96 * 3 * 128 * 2))
    assert f(2, 96, 3, 128, 128, 1, 1) == 0     # the plain call
    assert f(2, 96, 3, 128, 128, 1, 5) == 0     # 5 does not divide 96
    assert f(2, 96, 3, 96, 128, 1, 4) == 0
    assert f(2, 96, 3, 128, 128, 1, 0) == 0


@pytest.mark.parametrize("kw,code", [
    (dict(nseg=0), 1), (dict(nseg=5), 1), (dict(q=None), 1), (dict(ws=None), 1),
    (dict(ws=BAD), 1), (dict(wsb=100), 1), (dict(s0=BAD), 1), (dict(sf=BAD), 1),
    (dict(a=None), 1), (dict(o=None), 1), (dict(Dk=96), 2), (dict(dt=7), 2),
    (dict(flags=8), 2),
])
def test_split_validation(gdr, kw, code):
    assert split(gdr, **kw) == code


def test_split_empty(gdr):
    assert split(gdr, B=0, q=None, k=None, v=None, a=None, b=None, o=None, ws=None, wsb=0) == 0


def test_bwd_ex_flags(gdr):
    """The _ex backward calls reject unknown flag bits before anything else
    and take GDR_L2NORM_QK like the plain call otherwise (empty call)."""
    L = gdr.lib
    z = [None] * 20
    assert L.gdr_chunk_bwd_ex(0, 8, 1, 64, 64, 1, *z[:6], 1, *z[:2], *z[:6], None, 0, 2, None) == 2
    assert L.gdr_chunk_bwd_ex(0, 8, 1, 64, 64, 1, *z[:6], 1, *z[:2], *z[:6], None, 0, 1, None) == 0
    assert L.gdr2_chunk_bwd_ex(1, 8, 0, 64, 64, 1, *z[:7], 1, *z[:2], *z[:7], None, 0, 4,
                               None) == 2
    assert L.gdr2_chunk_bwd_ex(1, 8, 0, 64, 64, 1, *z[:7], 1, *z[:2], *z[:7], None, 0, 1,
                               None) == 0


def gate_bwd(gdr, N=4, H=2, Dv=64, odt=0, o=A16, gdt=1, g=A16, w=None, eps=1e-6, dyt=1, dy=A16,
             do=A16, dg=A16, dw=A16, ws=A16, wsb=None):
    if wsb is None:
        wsb = gdr.lib.gdr_output_gate_bwd_workspace_size(N, H, Dv)
    return gdr.lib.gdr_output_gate_bwd(N, H, Dv, odt, o, gdt, g, w, eps, dyt, dy, do, dg, dw, ws,
                                       wsb, None)


def test_gate_bwd_workspace_size(gdr):
    """Dv partial sums per workgroup, at most 2048 workgroups; a workgroup
    step takes 4 x 8 rows (Dv = 128) or 4 x 16 (Dv = 64)."""
    f = gdr.lib.gdr_output_gate_bwd_workspace_size
    assert f(100, 3, 128) == 4 * 128 * 10
    assert f(100, 3, 64) == 4 * 64 * 5
    assert f(10 ** 6, 16, 128) == 4 * 128 * 2048
    assert f(4, 2, 96) == 0


@pytest.mark.parametrize("kw,code", [
    (dict(o=None), 1), (dict(dy=BAD), 1), (dict(do=None), 1), (dict(dg=None), 1),
    (dict(w=BAD), 1), (dict(dw=BAD), 1), (dict(ws=None), 1), (dict(wsb=16), 1),
    (dict(eps=-1.0), 1), (dict(N=-1), 1), (dict(Dv=96), 2), (dict(dyt=3), 2),
])
def test_gate_bwd_validation(gdr, kw, code):
    assert gate_bwd(gdr, **kw) == code


def test_gate_bwd_no_workspace_without_dw(gdr):
    """dw NULL needs no workspace: only the pointer checks of the tensors
    remain (a misaligned dy is still rejected)."""
    assert gate_bwd(gdr, dw=None, ws=None, wsb=0, dy=BAD) == 1


def gate_bwd_noalloc(gdr, N=4, H=2, Dv=64, odt=0, o=A16, gdt=1, g=A16, w=None, eps=1e-6, dyt=1,
                     dy=A16, do=A16, dg=A16, dw=A16):
    return gdr.lib.gdr_output_gate_bwd_noalloc(N, H, Dv, odt, o, gdt, g, w, eps, dyt, dy, do, dg,
                                               dw, None)


@pytest.mark.parametrize("kw,code", [
    (dict(o=None), 1), (dict(dy=BAD), 1), (dict(do=None), 1), (dict(dg=None), 1),
    (dict(w=BAD), 1), (dict(dw=BAD), 1), (dict(eps=-1.0), 1), (dict(N=-1), 1),
    (dict(Dv=96), 2), (dict(dyt=3), 2), (dict(odt=5), 2),
])
def test_gate_bwd_noalloc_validation(gdr, kw, code):
    """The allocation-free gate backward rejects what gdr_output_gate_bwd
    rejects, on the host, before it touches the device."""
    assert gate_bwd_noalloc(gdr, **kw) == code


def test_gate_bwd_noalloc_scratch_limit():
    """The library's array holds the largest partial count the call can
    launch: 2048 workgroups x 128 channels of fp32, GDR_GATE_BWD_SCRATCH_BYTES
    in gdr.h."""
    hdr = open(HEADER).read()
    m = re.search(r"#define GDR_GATE_BWD_SCRATCH_BYTES \((\d+)u \* (\d+)u \* (\d+)u\)", hdr)
    assert m and int(m[1]) * int(m[2]) * int(m[3]) == 2048 * 128 * 4


def fwd_gate(gdr, B=2, T=5, H=2, Dk=64, Dv=64, dt=1, q=A16, k=A16, v=A16, a=A16, b=A16,
             s0=None, gdt=1, g=A16, w=None, eps=1e-6, odt=0, y=A16, sf=None, flags=0, ws=A16,
             wsb=None):
    if wsb is None:
        wsb = gdr.lib.gdr_chunk_fwd_gate_workspace_size(B, T, H, Dk, Dv, dt)
    return gdr.lib.gdr_chunk_fwd_gate(B, T, H, Dk, Dv, dt, q, k, v, a, b, s0, gdt, g, w, eps, odt,
                                      y, sf, flags, ws, wsb, None)


def test_fwd_gate_workspace_size(gdr):
    """bf16 inputs: per head, row block and one of four chunks, 32 words of 8
    bytes (16-row blocks when B H Dv / 64 < 128, else 64-row blocks); fp32
    inputs: an fp32 o; 0 for no tokens or unsupported sizes."""
    f = gdr.lib.gdr_chunk_fwd_gate_workspace_size
    assert f(8, 4096, 16, 128, 128, 1) == 8 * 16 * 2 * 4 * 32 * 8
    assert f(1, 100, 2, 128, 128, 1) == 2 * 8 * 4 * 32 * 8
    assert f(1, 100, 2, 128, 64, 1) == 2 * 4 * 4 * 32 * 8
    assert f(2, 10, 3, 64, 128, 0) == 2 * 10 * 3 * 128 * 4
    assert f(2, 0, 3, 64, 128, 1) == 0 and f(2, 10, 3, 96, 128, 1) == 0


@pytest.mark.parametrize("kw,code", [
    (dict(g=None), 1), (dict(g=BAD), 1), (dict(y=None), 1), (dict(w=BAD), 1),
    (dict(ws=None), 1), (dict(wsb=16), 1), (dict(eps=-1.0), 1), (dict(a=None), 1),
    (dict(Dv=96), 2), (dict(gdt=3), 2), (dict(odt=3), 2), (dict(flags=8), 2),
])
def test_fwd_gate_validation(gdr, kw, code):
    assert fwd_gate(gdr, **kw) == code


def test_bwd_split_workspace_size(gdr):
    """nseg = 1: the plain backward's workspace; otherwise the split
    forward's pieces (for fp32 inputs with the zero v and a discard buffer
    for the passes' outputs; the bf16 kernels need neither), N and the end
    gradients (fp32 per segment state), and the backward workspace of the
    segment batch; 0 where the call would reject the sizes."""
    f = gdr.lib.gdr_chunk_bwd_split_workspace_size
    up = lambda x: (x + 255) // 256 * 256
    assert f(2, 96, 3, 128, 128, 1, 1) == gdr.gdr_chunk_bwd_workspace_size(2, 96, 3, 128, 128)
    bn = 2 * 4 * 3
    fwd = up(bn * 128 * 128 * 4) * 3
    bw = up(gdr.gdr_chunk_bwd_workspace_size(8, 24, 3, 128, 128))
    assert f(2, 96, 3, 128, 128, 1, 4) == fwd + up(bn * 128 * 128 * 4) * 2 + bw
    fwd32 = fwd + up(2 * 96 * 3 * 128 * 4) + up(2 * 96 * 3 * 128 * 2)
    bw32 = up(gdr.gdr_chunk_bwd_workspace_size(8, 24, 3, 128, 128))
    assert f(2, 96, 3, 128, 128, 0, 4) == fwd32 + up(bn * 128 * 128 * 4) * 2 + bw32
    assert f(2, 96, 3, 128, 128, 1, 5) == 0
    assert f(2, 96, 3, 96, 128, 1, 4) == 0


@pytest.mark.parametrize("kw,code", [(dict(nseg=0), 1), (dict(nseg=7), 1), (dict(flags=4), 2),
                                     (dict(ws=None), 1), (dict(wsb=64), 1), (dict(ddt=9), 2)])
def test_bwd_split_validation(gdr, kw, code):
    nseg = kw.get("nseg", 4)
    flags = kw.get("flags", 0)
    wsb = kw.get("wsb", gdr.lib.gdr_chunk_bwd_split_workspace_size(1, 64, 1, 64, 64, 1,
                                                                     max(nseg, 1)))
    ws = kw.get("ws", A16)
    ddt = kw.get("ddt", 1)
    assert gdr.lib.gdr_chunk_bwd_split(1, 64, 1, 64, 64, 1, A16, A16, A16, A16, A16, None, ddt,
                                       A16, None, A16, A16, A16, A16, A16, None, nseg, flags, ws,
                                       wsb, None) == code


def test_head_count_bound(gdr):
    """The chunkwise calls take at most GDR_MAX_HEADS heads (their kernels
    address a chunk of tokens with 32-bit byte offsets): one more is
    rejected before anything is launched, the bound itself is accepted
    (B = 0, so nothing is launched either way)."""
    hdr = open(os.path.join(ROOT, "include", "gdr.h")).read()
    hmax = int(re.search(r"#define GDR_MAX_HEADS (\d+)", hdr).group(1))
    assert hmax == 65536
    for H, code in ((hmax, 0), (hmax + 1, 1)):
        assert chunk(gdr, B=0, H=H) == code
        assert chunk2(gdr, B=0, H=H) == code
        assert split(gdr, B=0, H=H, wsb=0) == code
        assert bwd(gdr, B=0, H=H, wsb=0) == code
        assert bwd2(gdr, B=0, H=H, wsb=0) == code
    big = hmax + 1
    assert gdr.gdr_chunk_bwd_workspace_size(1, 8, big, 64, 64) == 0
    assert gdr.gdr2_chunk_bwd_workspace_size(1, 8, big, 64, 64) == 0
    assert gdr.lib.gdr_chunk_fwd_split_workspace_size(1, 64, big, 64, 64, 1, 4) == 0
    assert gdr.gdr_chunk_bwd_workspace_size(1, 8, hmax, 64, 64) > 0


def test_split_fp32_states_flag(gdr):
    """GDR_SPLIT_FP32_STATES (2) is a gdr2_chunk_bwd_split bit only."""
    hdr = open(os.path.join(ROOT, "include", "gdr.h")).read()
    assert int(re.search(r"#define GDR_SPLIT_FP32_STATES (\d+)u", hdr).group(1)) == 2
    assert gdr.GDR_SPLIT_FP32_STATES == 2
    wsb = gdr.lib.gdr_chunk_bwd_split_workspace_size(1, 64, 1, 64, 64, 1, 4)
    assert gdr.lib.gdr_chunk_bwd_split(1, 64, 1, 64, 64, 1, A16, A16, A16, A16, A16, None, 1,
                                       A16, None, A16, A16, A16, A16, A16, None, 4, 2, A16,
                                       wsb, None) == 2
    assert split(gdr, flags=2) == 2
    wsb2 = gdr.lib.gdr2_chunk_bwd_split_workspace_size(1, 64, 1, 64, 64, 1, 4)
    call2 = lambda B, flags, n=4: gdr.lib.gdr2_chunk_bwd_split(
        B, 64, 1, 64, 64, 1, A16, A16, A16, A16, A16, A16, None, 1, A16, None, A16, A16, A16,
        A16, A16, A16, None, n, flags, A16, wsb2, None)
    assert call2(1, 2 | 4) == 2          # an unknown bit beside it
    assert call2(0, 2) == 0              # accepted (nothing to launch)
    assert call2(0, 2 | 1, n=1) == 0     # nseg = 1: ignored by the plain call


def _no_gpu():
    import torch
    return torch.cuda.device_count() == 0


@pytest.mark.skipif(not _no_gpu(), reason="calls that pass validation launch kernels on the "
                                          "fake addresses; host-only test")
def test_dispatch_work_item_bound(gdr):
    """One dispatch covers at most 2^32 - 1 work-items (workgroups x
    workgroup size).  Past the bound a call is rejected on the host
    (GDR_ERR_INVALID = 1) before anything is launched; at the bound it
    passes validation and reaches the launch, which fails here for want of
    a GPU (GDR_ERR_DEVICE = 3).  Bounds: 2^21 - 8 heads in a chunkwise call
    (2048 work-items per head on a grid rounded up to 8 heads), 2^24 - 1
    (sequence, head) pairs in a decode step (256 each), 2^32 - 256 elements
    B T H Dk in a backward (one work-item per element)."""
    heads = (1 << 21) - 8
    assert chunk(gdr, B=heads, T=1) == 3
    assert chunk(gdr, B=heads + 1, T=1) == 1
    assert chunk2(gdr, B=heads, T=1) == 3
    assert chunk2(gdr, B=heads + 1, T=1) == 1
    assert split(gdr, B=heads // 4, T=4, nseg=4, wsb=1 << 60) == 3
    assert split(gdr, B=heads // 4 + 1, T=4, nseg=4, wsb=1 << 60) == 1
    assert step(gdr, N=(1 << 24) - 1) == 3
    assert step(gdr, N=1 << 24) == 1
    assert step(gdr, N=1 << 23, H=2) == 1
    elems = (1 << 32) - 256                     # B T H Dk with Dk = 64
    assert bwd(gdr, T=elems // 64, wsb=1 << 60) == 3
    assert bwd(gdr, T=elems // 64 + 1, wsb=1 << 60) == 1
    assert bwd2(gdr, T=elems // 64, wsb=1 << 60) == 3
    assert bwd2(gdr, T=elems // 64 + 1, wsb=1 << 60) == 1


def test_gdr2_bwd_split_workspace_covers_plain(gdr):
    """GDR_SPLIT_FP32_STATES runs the plain backward in the split call's
    workspace, so the split size covers the plain one."""
    f = gdr.lib.gdr2_chunk_bwd_split_workspace_size
    for B, T, H, nseg in ((1, 64, 2, 4), (2, 90, 1, 3), (1, 32768, 16, 4)):
        assert f(B, T, H, 128, 128, 1, nseg) >= gdr.gdr2_chunk_bwd_workspace_size(B, T, H, 128,
                                                                                   128)
