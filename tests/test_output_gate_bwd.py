"""GPU parity of gdr_output_gate_bwd (reverse mode of the RMSNorm x SiLU
output gate) against the oracle's reverse mode on the same seeded inputs
and output gradients.  Metric: max error over rms per gradient, 1e-3 (fp32
arithmetic on exact inputs)."""
import numpy as np
import pytest
import torch

import oracle
from gdr_gen import make_gate

pytestmark = pytest.mark.gpu

DT = {"f32": torch.float32, "bf16": torch.bfloat16}
TOL = 1e-3


def _check(gdr_lib, inp, eps, dy_dt="f32", seed=0):
    print(f"gate bwd {inp.meta} eps={eps} dy={dy_dt}", flush=True)
    g = np.random.Generator(np.random.PCG64(seed))
    dy = torch.from_numpy(g.standard_normal(tuple(inp.o.shape)).astype(np.float32)).to(DT[dy_dt])
    ref = oracle.rmsnorm_gate_bwd(inp.o, inp.g, inp.w, dy, eps=eps)
    w = None if inp.w is None else inp.w.cuda()
    got = gdr_lib.gdr_output_gate_bwd(inp.o.cuda(), inp.g.cuda(), w, dy.cuda(), eps)
    torch.cuda.synchronize()
    names = ("do", "dg", "dw")
    errs = {}
    for n, x, y in zip(names, got, ref):
        if y is None:
            continue
        errs[n] = oracle.err_rms(x.cpu(), y)
    print("  " + " ".join(f"{n}={e:.2e}" for n, e in errs.items()))
    bad = {n: e for n, e in errs.items() if not e <= TOL}
    assert not bad, bad


@pytest.mark.parametrize("N", [1, 7, 100, 4097])
@pytest.mark.parametrize("Dv", [64, 128])
def test_gate_bwd_ragged(gdr_lib, N, Dv):
    _check(gdr_lib, make_gate(N, 3, Dv, "f32", "bf16", seed=420 + N + Dv), 1e-6, seed=N)


@pytest.mark.parametrize("odt,gdt,dyt", [("f32", "f32", "f32"), ("bf16", "bf16", "bf16"),
                                         ("f32", "bf16", "bf16"), ("bf16", "f32", "f32")])
@pytest.mark.parametrize("weight", [True, False])
def test_gate_bwd_dtypes(gdr_lib, odt, gdt, dyt, weight):
    _check(gdr_lib, make_gate(300, 4, 128, odt, gdt, seed=430, weight=weight), 1e-6, dyt, 1)


@pytest.mark.parametrize("eps", [0.0, 1e-2])
def test_gate_bwd_eps(gdr_lib, eps):
    _check(gdr_lib, make_gate(200, 2, 64, "f32", "f32", seed=440), eps, seed=2)


def test_gate_bwd_without_dw(gdr_lib):
    """dw not wanted: no workspace; do and dg as before."""
    inp = make_gate(50, 2, 128, "f32", "bf16", seed=450)
    dy = torch.randn(tuple(inp.o.shape))
    do, dg, dw = gdr_lib.gdr_output_gate_bwd(inp.o.cuda(), inp.g.cuda(), inp.w.cuda(), dy.cuda(),
                                             want_dw=False)
    torch.cuda.synchronize()
    assert dw is None
    ref = oracle.rmsnorm_gate_bwd(inp.o, inp.g, inp.w, dy)
    assert oracle.err_rms(do.cpu(), ref[0]) <= TOL and oracle.err_rms(dg.cpu(), ref[1]) <= TOL


def test_gate_bwd_workload(gdr_lib):
    """The B8 T4096 H16 d128 gate (fp32 o, bf16 gate and dy): 524,288 rows,
    dw summed over all of them by 1024 workgroups."""
    inp = make_gate(8 * 4096, 16, 128, "f32", "bf16", seed=1005)
    _check(gdr_lib, inp, 1e-6, "bf16", 3)
