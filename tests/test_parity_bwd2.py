"""GPU parity of gdr2_chunk_bwd (reverse mode of Gated Delta Rule-2) against
the fp64 oracle's token-by-token backward on the same seeded inputs and
output gradients.  Metric per gradient: max error over rms, 1e-3 (the
kernels compute in fp32 on exact inputs, fp32 or bf16)."""
import numpy as np
import pytest
import torch

import oracle
from gdr_gen import make_gdn2

pytestmark = pytest.mark.gpu

TOL = 1e-3
NAMES = ("dq", "dk", "dv", "dalpha", "derase", "dwrite", "ds0")


def _grads_in(inp, dout_dtype, seed, with_dsf=True):
    g = np.random.Generator(np.random.PCG64(seed))
    B, T, H, Dk = inp.q.shape
    Dv = inp.v.shape[-1]
    do = torch.from_numpy(g.standard_normal((B, T, H, Dv)).astype(np.float32)).to(dout_dtype)
    dsf = (torch.from_numpy((0.1 * g.standard_normal((B, H, Dv, Dk))).astype(np.float32))
           if with_dsf else None)
    return do, dsf


def _args(inp):
    return (inp.q, inp.k, inp.v, inp.alpha, inp.erase, inp.write, inp.s0)


def _check(gdr_lib, inp, dout_dtype=torch.float32, seed=0, with_dsf=True, tol=TOL,
           log_alpha=False):
    """``log_alpha``: compare alpha * dalpha, the gradient with respect to
    log alpha, instead of dalpha.  The chunked form obtains dalpha as that
    gradient over alpha, so where alpha is near 0 its absolute error grows
    like 1 / alpha (the gradient with respect to log alpha keeps fp32
    accuracy); the oracle differentiates alpha itself."""
    print(f"bwd2 {inp.meta} dout={dout_dtype} dsf={with_dsf}", flush=True)
    do, dsf = _grads_in(inp, dout_dtype, seed, with_dsf)
    ref = oracle.gdn2_bwd(*_args(inp), do, dsf)
    c = lambda x: None if x is None else x.cuda()
    got = gdr_lib.gdr2_chunk_bwd(*[c(x) for x in _args(inp)], c(do), c(dsf))
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


@pytest.mark.parametrize("T", [1, 15, 16, 17, 100, 257])
def test_bwd2_fp32_ragged(gdr_lib, T):
    _check(gdr_lib, make_gdn2(B=1, T=T, H=2, Dk=64, Dv=64, dtype="f32", seed=600 + T,
                              s0_std=0.5), seed=T)


@pytest.mark.parametrize("dims", [(128, 128), (128, 64), (64, 128), (64, 64)])
def test_bwd2_dims(gdr_lib, dims):
    _check(gdr_lib, make_gdn2(B=2, T=70, H=2, Dk=dims[0], Dv=dims[1], dtype="f32",
                              seed=610 + dims[0] + dims[1], s0_std=0.2), seed=1)


@pytest.mark.parametrize("dout", ["f32", "bf16"])
def test_bwd2_bf16_inputs(gdr_lib, dout):
    dt = torch.bfloat16 if dout == "bf16" else torch.float32
    _check(gdr_lib, make_gdn2(B=1, T=150, H=3, Dk=128, Dv=128, dtype="bf16", seed=620,
                              s0_std=0.05), dout_dtype=dt, seed=2)


def test_bwd2_no_state_gradients(gdr_lib):
    """No S_0 and no dL/dS_T: only the output carries gradient."""
    _check(gdr_lib, make_gdn2(B=2, T=90, H=2, Dk=128, Dv=64, dtype="f32", seed=630),
           seed=3, with_dsf=False)


def test_bwd2_gate_regimes(gdr_lib):
    """Long memory (alpha near 1), erase strengths up to 2 and single channels
    that reset (alpha = 0 and 1e-12): the decay tables must stay finite."""
    inp = make_gdn2(B=1, T=120, H=2, Dk=64, Dv=64, dtype="f32", seed=640, alpha_shift=-4.0,
                    s0_std=0.2)
    inp.erase = inp.erase * 2.0
    a = inp.alpha.clone()
    a[0, 20:23, 0, 5] = 1e-12
    a[0, 70, 1, :] = 0.0
    inp.alpha = a
    _check(gdr_lib, inp, seed=4, log_alpha=True)


def test_bwd2_workload(gdr_lib):
    """The B4 H16 T4096 d128 bf16 workload with bf16 output gradients,
    every gradient of every head against the oracle.

    The alpha gradient is compared as d log alpha = alpha (.) dL/dalpha:
    the rule's chunk form runs on cumulative log decays, and the kernel
    forms d log alpha and divides by alpha last.  Over this workload's 33M
    per-channel gates alpha reaches 6e-4, where the quotient multiplies the
    fp32 rounding of d log alpha (6.6e-5 of its rms here) by up to 1.7e3, so
    the max/rms metric of dL/dalpha itself measures the far tail of the gate
    distribution (1.2e-3 on two of the 64 heads) rather than the kernel.
    The small-shape cases above compare dL/dalpha directly."""
    inp = make_gdn2(B=4, T=4096, H=16, Dk=128, Dv=128, dtype="bf16", seed=1004)
    do, dsf = _grads_in(inp, torch.bfloat16, 5)
    print("bwd2 B4 H16 T4096", flush=True)
    got = gdr_lib.gdr2_chunk_bwd(*[None if x is None else x.cuda() for x in _args(inp)],
                                 do.cuda(), dsf.cuda())
    torch.cuda.synchronize()
    ref = oracle.gdn2_bwd(*_args(inp), do, dsf)
    alpha = inp.alpha.double().numpy()
    for name, x, y in zip(NAMES, got, ref):
        x = x.cpu()
        if name == "dalpha":
            x, y = x.double().numpy() * alpha, y * alpha
        e = oracle.err_rms(x, y)
        print(f"  {name}={e:.2e}")
        assert e <= TOL, (name, e)
