"""GPU parity of gdr_chunk_bwd (reverse mode of the scalar-gate rule)
against the fp64 oracle's token-by-token backward on the same seeded inputs
and output gradients.  Metric per gradient: max error over rms, 1e-3 (the
kernels compute in fp32 on exact inputs, fp32 or bf16)."""
import numpy as np
import pytest
import torch

import oracle
from gdr_gen import make_gdn

pytestmark = pytest.mark.gpu

TOL = 1e-3
NAMES = ("dq", "dk", "dv", "dalpha", "dbeta", "ds0")


def _grads_in(inp, dout_dtype, seed, with_dsf=True):
    g = np.random.Generator(np.random.PCG64(seed))
    B, T, H, Dk = inp.q.shape
    Dv = inp.v.shape[-1]
    do = torch.from_numpy(g.standard_normal((B, T, H, Dv)).astype(np.float32)).to(dout_dtype)
    dsf = (torch.from_numpy((0.1 * g.standard_normal((B, H, Dv, Dk))).astype(np.float32))
           if with_dsf else None)
    return do, dsf


def _check(gdr_lib, inp, dout_dtype=torch.float32, seed=0, with_dsf=True, tol=TOL,
           log_alpha=False):
    """``log_alpha``: compare alpha * dalpha (the gradient with respect to
    log alpha, which keeps fp32 accuracy where alpha is near 0; the kernels
    divide it by alpha) instead of dalpha."""
    print(f"bwd {inp.meta} dout={dout_dtype} dsf={with_dsf}", flush=True)
    do, dsf = _grads_in(inp, dout_dtype, seed, with_dsf)
    ref = oracle.gdn_bwd(inp.q, inp.k, inp.v, inp.alpha, inp.beta, inp.s0, do, dsf)
    c = lambda x: None if x is None else x.cuda()
    got = gdr_lib.gdr_chunk_bwd(c(inp.q), c(inp.k), c(inp.v), c(inp.alpha), c(inp.beta),
                                c(inp.s0), c(do), c(dsf))
    torch.cuda.synchronize()
    errs = {}
    for name, x, y in zip(NAMES, got, ref):
        x = x.cpu()
        if log_alpha and name == "dalpha":
            a = inp.alpha.double().numpy()
            x, y = x.double().numpy() * a, y * a
        errs[name] = oracle.err_rms(x, y)
    print("  " + " ".join(f"{n}={e:.2e}" for n, e in errs.items()))
    bad = {n: e for n, e in errs.items() if not e <= tol}
    assert not bad, bad
    return errs


@pytest.mark.parametrize("T", [1, 31, 32, 33, 100, 257])
def test_bwd_fp32_ragged(gdr_lib, T):
    _check(gdr_lib, make_gdn(B=1, T=T, H=2, Dk=64, Dv=64, dtype="f32", seed=500 + T,
                             s0_std=0.5), seed=T)


@pytest.mark.parametrize("dims", [(128, 128), (128, 64), (64, 128), (64, 64)])
def test_bwd_dims(gdr_lib, dims):
    _check(gdr_lib, make_gdn(B=2, T=70, H=2, Dk=dims[0], Dv=dims[1], dtype="f32",
                             seed=510 + dims[0] + dims[1], s0_std=0.2), seed=1)


@pytest.mark.parametrize("dout", ["f32", "bf16"])
def test_bwd_bf16_inputs(gdr_lib, dout):
    dt = torch.bfloat16 if dout == "bf16" else torch.float32
    _check(gdr_lib, make_gdn(B=1, T=150, H=3, Dk=128, Dv=128, dtype="bf16", seed=520,
                             s0_std=0.05), dout_dtype=dt, seed=2)


def test_bwd_no_state_gradients(gdr_lib):
    """No S_0 and no dL/dS_T: only the output carries gradient."""
    _check(gdr_lib, make_gdn(B=2, T=90, H=2, Dk=128, Dv=64, dtype="f32", seed=530),
           seed=3, with_dsf=False)


def test_bwd_gate_regimes(gdr_lib):
    """Long memory (alpha near 1) and beta up to 2 (negative eigenvalues)."""
    inp = make_gdn(B=1, T=200, H=2, Dk=64, Dv=64, dtype="f32", seed=540, alpha_shift=-4.0,
                   s0_std=0.2)
    inp.beta = inp.beta * 2.0
    _check(gdr_lib, inp, seed=4)


def test_bwd_reset_gates(gdr_lib):
    """alpha = 0 and 1e-12 on some tokens: the within-chunk decays across them
    underflow to 0 (every decay the kernel forms is at most 1)."""
    inp = make_gdn(B=1, T=130, H=2, Dk=64, Dv=64, dtype="f32", seed=545, s0_std=0.2)
    a = inp.alpha.clone()
    a[0, 20, 0] = 0.0
    a[0, 57:60, 1] = 1e-12
    a[0, 129, 0] = 0.0
    inp.alpha = a
    _check(gdr_lib, inp, seed=6, log_alpha=True)


def test_bwd_workload(gdr_lib):
    """The B8 H16 T4096 d128 bf16 workload with bf16 output gradients,
    every gradient of every head against the oracle."""
    inp = make_gdn(B=8, T=4096, H=16, Dk=128, Dv=128, dtype="bf16", seed=1001)
    do, dsf = _grads_in(inp, torch.bfloat16, 5)
    print("bwd B8 H16 T4096", flush=True)
    got = gdr_lib.gdr_chunk_bwd(inp.q.cuda(), inp.k.cuda(), inp.v.cuda(), inp.alpha.cuda(),
                                inp.beta.cuda(), None, do.cuda(), dsf.cuda())
    torch.cuda.synchronize()
    ref = oracle.gdn_bwd(inp.q, inp.k, inp.v, inp.alpha, inp.beta, None, do, dsf)
    for name, x, y in zip(NAMES, got, ref):
        e = oracle.err_rms(x.cpu(), y)
        print(f"  {name}={e:.2e}")
        assert e <= TOL, (name, e)
