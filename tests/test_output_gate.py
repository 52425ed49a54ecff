"""GPU parity of gdr_output_gate (RMSNorm of the rule's output times a SiLU
gate) against the fp64 oracle on the same seeded inputs.  Metric: max error
over rms(y), 1e-3 (fp32 arithmetic on exact inputs), plus half a bf16 ulp per
element measured on the oracle's output when y is bf16."""
import numpy as np
import pytest
import torch

import oracle
from gdr_gen import make_gate

pytestmark = pytest.mark.gpu

DT = {"f32": torch.float32, "bf16": torch.bfloat16}


def _tol(y_ref, out):
    t = 1e-3
    if out == "bf16":
        yb = torch.from_numpy(np.asarray(y_ref, dtype=np.float32)).to(torch.bfloat16)
        t += oracle.err_rms(yb.double().numpy(), y_ref)
    return t


def _check(gdr_lib, inp, eps, out, inplace=False):
    print(f"output gate {inp.meta} eps={eps} out={out} inplace={inplace}", flush=True)
    y_ref = oracle.rmsnorm_gate(inp.o, inp.g, inp.w, eps=eps)
    o = inp.o.cuda()
    w = None if inp.w is None else inp.w.cuda()
    if inplace:
        y = gdr_lib.gdr_output_gate(o, inp.g.cuda(), w, eps, y=o)
        assert y is o
    else:
        y = gdr_lib.gdr_output_gate(o, inp.g.cuda(), w, eps, out_dtype=DT[out])
    torch.cuda.synchronize()
    e = oracle.err_rms(y.cpu(), y_ref)
    assert e <= _tol(y_ref, out), e
    return e


@pytest.mark.parametrize("N", [1, 7, 100, 4097])
@pytest.mark.parametrize("Dv", [64, 128])
def test_gate_ragged(gdr_lib, N, Dv):
    _check(gdr_lib, make_gate(N, 3, Dv, "f32", "bf16", seed=400 + N + Dv), 1e-6, "bf16")


@pytest.mark.parametrize("odt,gdt,out", [("f32", "f32", "f32"), ("f32", "bf16", "bf16"),
                                         ("bf16", "bf16", "bf16"), ("bf16", "f32", "f32"),
                                         ("f32", "bf16", "f32")])
@pytest.mark.parametrize("weight", [True, False])
def test_gate_dtypes(gdr_lib, odt, gdt, out, weight):
    _check(gdr_lib, make_gate(333, 4, 128, odt, gdt, seed=410, weight=weight), 1e-6, out)


@pytest.mark.parametrize("eps", [0.0, 1e-6, 1e-2, 1.0])
def test_gate_eps(gdr_lib, eps):
    _check(gdr_lib, make_gate(200, 2, 64, "f32", "f32", seed=420), eps, "f32")


@pytest.mark.parametrize("odt", ["f32", "bf16"])
def test_gate_in_place(gdr_lib, odt):
    _check(gdr_lib, make_gate(517, 2, 128, odt, "bf16", seed=430), 1e-6, odt, inplace=True)


def test_gate_zero_rows_and_saturated_gates(gdr_lib):
    """Zero rows give zero (eps keeps them finite); gates of +-60 give SiLU
    of 60 and ~0 (no overflow in the exponential)."""
    inp = make_gate(64, 2, 128, "f32", "f32", seed=440)
    o, g = inp.o.clone(), inp.g.clone()
    o[3] = 0
    o[10, 1] = 0
    g[20, 0, :64] = 60.0
    g[21, 1, 64:] = -60.0
    inp.o, inp.g = o, g
    _check(gdr_lib, inp, 1e-6, "f32")


def test_gate_workload_b8_t4096_h16(gdr_lib):
    """The output of the scalar-gate workload (B8 T4096 H16 Dv128, fp32 o,
    bf16 gate, bf16 y); the oracle checks the first and last 2048 tokens."""
    inp = make_gate(8 * 4096, 16, 128, "f32", "bf16", seed=450)
    print("output gate B8 T4096 H16", flush=True)
    y = gdr_lib.gdr_output_gate(inp.o.cuda(), inp.g.cuda(), inp.w.cuda(), 1e-6,
                                out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    y = y.cpu()
    for sl in (slice(0, 2048), slice(-2048, None)):
        y_ref = oracle.rmsnorm_gate(inp.o[sl], inp.g[sl], inp.w, eps=1e-6)
        e = oracle.err_rms(y[sl], y_ref)
        assert e <= _tol(y_ref, "bf16"), e
