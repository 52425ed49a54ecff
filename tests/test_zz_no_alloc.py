"""gdr_output_gate_bwd_noalloc, the gate backward that takes no workspace,
against gdr_output_gate_bwd (the call with a caller workspace) on the same
inputs: both run the same kernels over the same partial count, so the
results must agree bit for bit.  Two calls in a row, the second on a smaller
input, so the second reuses the library's array after the first filled it;
each call is also checked against the oracle at the fp32 tolerance."""
import numpy as np
import pytest
import torch

import oracle
from gdr_gen import make_gate

pytestmark = pytest.mark.gpu

DT = {"f32": torch.float32, "bf16": torch.bfloat16}


def _dy(shape, dt, seed):
    g = np.random.Generator(np.random.PCG64(seed))
    return torch.from_numpy(g.standard_normal(shape).astype(np.float32)).to(DT[dt])


def _one(gdr_lib, N, H, Dv, odt, gdt, dyt, seed, eps=1e-6):
    print(f"noalloc gate bwd N={N} H={H} Dv={Dv} o={odt} g={gdt} dy={dyt}", flush=True)
    inp = make_gate(N, H, Dv, odt, gdt, seed=seed)
    dy = _dy(tuple(inp.o.shape), dyt, seed + 1)
    o, g, d = inp.o.cuda(), inp.g.cuda(), dy.cuda()
    w = None if inp.w is None else inp.w.cuda()
    ref = gdr_lib.gdr_output_gate_bwd(o, g, w, d, eps)
    got = gdr_lib.gdr_output_gate_bwd_noalloc(o, g, w, d, eps)
    torch.cuda.synchronize()
    for name, x, y in zip(("do", "dg", "dw"), got, ref):
        assert torch.equal(x, y), f"{name} differs from gdr_output_gate_bwd"
    want = oracle.rmsnorm_gate_bwd(inp.o, inp.g, inp.w, dy, eps=eps)
    for name, x, y in zip(("do", "dg", "dw"), got, want):
        e = oracle.err_rms(x.cpu(), y)
        assert e <= 1e-3, f"{name}: {e:.2e}"


@pytest.mark.parametrize("Dv", [64, 128])
def test_noalloc_two_calls_second_smaller(gdr_lib, Dv):
    # the first call fills every partial the kernel launches (the cap of
    # 2048 workgroups), the second reads back only its own, fewer ones
    _one(gdr_lib, 40000, 4, Dv, "f32", "bf16", "bf16", seed=900 + Dv)
    _one(gdr_lib, 37, 3, Dv, "bf16", "f32", "f32", seed=910 + Dv)


def test_noalloc_without_dw(gdr_lib):
    inp = make_gate(50, 2, 128, "f32", "f32", seed=920)
    dy = _dy(tuple(inp.o.shape), "f32", 921).cuda()
    o, g = inp.o.cuda(), inp.g.cuda()
    w = inp.w.cuda()
    ref = gdr_lib.gdr_output_gate_bwd(o, g, w, dy, 1e-6, want_dw=False)
    got = gdr_lib.gdr_output_gate_bwd_noalloc(o, g, w, dy, 1e-6, want_dw=False)
    torch.cuda.synchronize()
    assert got[2] is None
    assert torch.equal(got[0], ref[0]) and torch.equal(got[1], ref[1])


def test_noalloc_empty_rows_zero_dw(gdr_lib):
    o = torch.empty((0, 2, 64), device="cuda")
    _, _, dw = gdr_lib.gdr_output_gate_bwd_noalloc(o, o.clone(), None, o.clone(), 1e-6)
    torch.cuda.synchronize()
    assert torch.count_nonzero(dw).item() == 0
