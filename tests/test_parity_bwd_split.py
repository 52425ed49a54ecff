"""GPU parity of gdr_chunk_bwd_split (the backward over segments side by
side, composed through the carry's affine map) against the oracle's
backward, at the plain backward's tolerance (1e-3 of rms per gradient)."""
import numpy as np
import pytest
import torch

import oracle
from gdr_gen import make_gdn

pytestmark = pytest.mark.gpu

TOL = 1e-3
NAMES = ("dq", "dk", "dv", "dalpha", "dbeta", "ds0")


def _check(gdr_lib, inp, nseg, seed, dout_dtype=torch.float32, norm=False, with_dsf=True):
    print(f"bwd split nseg={nseg} {inp.meta} norm={norm}", flush=True)
    g = np.random.Generator(np.random.PCG64(seed))
    B, T, H, Dk = inp.q.shape
    Dv = inp.v.shape[-1]
    do = torch.from_numpy(g.standard_normal((B, T, H, Dv)).astype(np.float32)).to(dout_dtype)
    dsf = (torch.from_numpy((0.1 * g.standard_normal((B, H, Dv, Dk))).astype(np.float32))
           if with_dsf else None)
    qn = torch.from_numpy(oracle.l2norm(inp.q)) if norm else inp.q
    kn = torch.from_numpy(oracle.l2norm(inp.k)) if norm else inp.k
    ref = list(oracle.gdn_bwd(qn, kn, inp.v, inp.alpha, inp.beta, inp.s0, do, dsf))
    if norm:
        ref[0], ref[1] = oracle.l2norm_bwd(inp.q, ref[0]), oracle.l2norm_bwd(inp.k, ref[1])
    c = lambda x: None if x is None else x.cuda()
    got = gdr_lib.gdr_chunk_bwd_split(c(inp.q), c(inp.k), c(inp.v), c(inp.alpha), c(inp.beta),
                                      c(inp.s0), c(do), c(dsf), nseg=nseg, l2norm_qk=norm)
    torch.cuda.synchronize()
    errs = {n: oracle.err_rms(x.cpu(), y) for n, x, y in zip(NAMES, got, ref)}
    print("  " + " ".join(f"{n}={e:.2e}" for n, e in errs.items()))
    bad = {n: e for n, e in errs.items() if not e <= TOL}
    assert not bad, bad


@pytest.mark.parametrize("nseg", [2, 4, 8])
def test_bwd_split_long_memory(gdr_lib, nseg):
    """alpha near 1: the carry through P^T matters."""
    _check(gdr_lib, make_gdn(B=1, T=256, H=2, Dk=128, Dv=128, dtype="f32", seed=760 + nseg,
                             alpha_shift=-4.0, s0_std=0.1), nseg, nseg)


@pytest.mark.parametrize("nseg", [3, 5])
def test_bwd_split_ragged_segments(gdr_lib, nseg):
    """Segments of 30 and 18 tokens (not multiples of the 16-token chunk)."""
    _check(gdr_lib, make_gdn(B=2, T=90, H=2, Dk=64, Dv=64, dtype="f32", seed=770 + nseg,
                             alpha_shift=-1.0, s0_std=0.2), nseg, 10 + nseg)


@pytest.mark.parametrize("dims", [(128, 64), (64, 128)])
def test_bwd_split_dims(gdr_lib, dims):
    _check(gdr_lib, make_gdn(B=1, T=128, H=3, Dk=dims[0], Dv=dims[1], dtype="f32",
                             seed=780 + dims[0], alpha_shift=-2.0, s0_std=0.1), 4, 20)


@pytest.mark.parametrize("dims", [(128, 64), (64, 128), (64, 64)])
def test_bwd_split_bf16_dims(gdr_lib, dims):
    """bf16 inputs: the transition pass reads no v (d_v of that pass = d_k)
    and the scans run at every head-dim pair."""
    _check(gdr_lib, make_gdn(B=1, T=160, H=2, Dk=dims[0], Dv=dims[1], dtype="bf16",
                             seed=785 + dims[0] + dims[1], alpha_shift=-2.0, s0_std=0.1), 5,
           22, dout_dtype=torch.bfloat16)


def test_bwd_split_bf16_norm_no_state(gdr_lib):
    """bf16 inputs and dL/do, q, k normalised on load, no S_0 or dL/dS_T."""
    _check(gdr_lib, make_gdn(B=1, T=192, H=2, Dk=128, Dv=128, dtype="bf16", seed=790,
                             alpha_shift=-3.0, raw_qk=True), 4, 21, dout_dtype=torch.bfloat16,
           norm=True, with_dsf=False)


def test_bwd_split_one_segment_is_plain(gdr_lib):
    inp = make_gdn(B=1, T=64, H=2, Dk=64, Dv=64, dtype="f32", seed=795, s0_std=0.1)
    do = torch.randn((1, 64, 2, 64))
    args = [x.cuda() for x in (inp.q, inp.k, inp.v, inp.alpha, inp.beta, inp.s0)] + [do.cuda()]
    a = gdr_lib.gdr_chunk_bwd(*args)
    b = gdr_lib.gdr_chunk_bwd_split(*args, nseg=1)
    torch.cuda.synchronize()
    # dq and dk are sums over row blocks by atomic adds, whose order varies
    # from run to run: equal to fp32 rounding; the rest bit for bit
    for name, x, y in zip(NAMES, a, b):
        if name in ("dq", "dk"):
            assert ((x - y).abs().max() <= 1e-5 * x.abs().max()).item(), name
        else:
            assert torch.equal(x, y), name


def test_bwd_split_long_context_workload(gdr_lib):
    """The long-context backward the benchmark times: B1 H16 T32768 d128,
    bf16 inputs and dL/do, an initial state and dL/dS_T, in 4 segments;
    every head against the oracle (it keeps segment checkpoints, so the
    whole sequence fits)."""
    from gdr_gen import make_config
    _check(gdr_lib, make_config(2), 4, 22, dout_dtype=torch.bfloat16)


def test_gdr2_split_long_context_workload(gdr_lib):
    """Gated Delta Rule-2 at the same shape (per-channel alpha near 1), as
    timed: the split forward's o and final state, then the split backward,
    every head against the oracle.  The backward's segment start states
    come from the forward with every computed operand split (hi/lo), so
    every gradient is held to 1e-3; with GDR_SPLIT_FP32_STATES the call is
    the plain backward, held to the same."""
    from gdr_gen import make_gdn2
    inp = make_gdn2(B=1, T=32768, H=16, Dk=128, Dv=128, dtype="bf16", seed=1006,
                    alpha_shift=-4.0, s0_std=0.02)
    args = (inp.q, inp.k, inp.v, inp.alpha, inp.erase, inp.write, inp.s0)
    print(f"gdr2 split long context {inp.meta}", flush=True)
    c = lambda x: None if x is None else x.cuda()
    o, s = gdr_lib.gdr2_chunk_fwd_split(*map(c, args), nseg=4, out_dtype=torch.float32)
    torch.cuda.synchronize()
    o_ref, s_ref = oracle.gdn2_fwd(*args)
    eo, es = oracle.err_rms(o.cpu(), o_ref), oracle.err_rms(s.cpu(), s_ref)
    print(f"  fwd err(o)={eo:.2e} err(S)={es:.2e}")
    assert eo <= 2e-2 and es <= 2e-2, (eo, es)
    g = np.random.Generator(np.random.PCG64(23))
    do = torch.from_numpy(g.standard_normal((1, 32768, 16, 128)).astype(np.float32)).to(
        torch.bfloat16)
    dsf = torch.from_numpy((0.1 * g.standard_normal((1, 16, 128, 128))).astype(np.float32))
    ref = oracle.gdn2_bwd(*args, do, dsf)
    names = ("dq", "dk", "dv", "dalpha", "derase", "dwrite", "ds0")
    for fp32_states in (False, True):
        got = gdr_lib.gdr2_chunk_bwd_split(*map(c, args), c(do), c(dsf), nseg=4,
                                           fp32_states=fp32_states)
        torch.cuda.synchronize()
        errs = {n: oracle.err_rms(x.cpu(), y) for n, x, y in zip(names, got, ref)}
        print(f"  bwd fp32_states={fp32_states} " +
              " ".join(f"{n}={e:.2e}" for n, e in errs.items()))
        bad = {n: e for n, e in errs.items() if not e <= TOL}
        assert not bad, (fp32_states, bad)


NAMES2 = ("dq", "dk", "dv", "dalpha", "derase", "dwrite", "ds0")


def _check2(gdr_lib, inp, nseg, seed, norm=False):
    """gdr2_chunk_bwd_split (bf16 inputs and dL/do) against the oracle's
    backward of Gated Delta Rule-2, every gradient at 1e-3."""
    print(f"gdr2 bwd split nseg={nseg} {inp.meta} norm={norm}", flush=True)
    g = np.random.Generator(np.random.PCG64(seed))
    B, T, H, Dk = inp.q.shape
    Dv = inp.v.shape[-1]
    do = torch.from_numpy(g.standard_normal((B, T, H, Dv)).astype(np.float32)).to(torch.bfloat16)
    dsf = torch.from_numpy((0.1 * g.standard_normal((B, H, Dv, Dk))).astype(np.float32))
    qn = torch.from_numpy(oracle.l2norm(inp.q)) if norm else inp.q
    kn = torch.from_numpy(oracle.l2norm(inp.k)) if norm else inp.k
    ref = list(oracle.gdn2_bwd(qn, kn, inp.v, inp.alpha, inp.erase, inp.write, inp.s0, do, dsf))
    if norm:
        ref[0], ref[1] = oracle.l2norm_bwd(inp.q, ref[0]), oracle.l2norm_bwd(inp.k, ref[1])
    c = lambda x: None if x is None else x.cuda()
    args = [c(x) for x in (inp.q, inp.k, inp.v, inp.alpha, inp.erase, inp.write, inp.s0)]
    got = gdr_lib.gdr2_chunk_bwd_split(*args, c(do), c(dsf), nseg=nseg, l2norm_qk=norm)
    plain = gdr_lib.gdr2_chunk_bwd(*args, c(do), c(dsf), l2norm_qk=norm)
    flag = gdr_lib.gdr2_chunk_bwd_split(*args, c(do), c(dsf), nseg=nseg, l2norm_qk=norm,
                                        fp32_states=True)
    torch.cuda.synchronize()
    errs = {n: oracle.err_rms(x.cpu(), y) for n, x, y in zip(NAMES2, got, ref)}
    print("  " + " ".join(f"{n}={e:.2e}" for n, e in errs.items()))
    bad = {n: e for n, e in errs.items() if not e <= TOL}
    assert not bad, bad
    # GDR_SPLIT_FP32_STATES is the plain call: dq, dk, derase and dalpha are
    # sums over row blocks by atomic adds, whose order varies from run to
    # run (equal to fp32 rounding); the rest bit for bit
    for n, x, y in zip(NAMES2, flag, plain):
        if n in ("dq", "dk", "dalpha", "derase"):
            assert ((x - y).abs().max() <= 1e-5 * x.abs().max()).item(), n
        else:
            assert torch.equal(x, y), n


@pytest.mark.parametrize("dims", [(128, 64), (64, 128), (128, 128)])
def test_gdr2_bwd_split_dims(gdr_lib, dims):
    """Per-channel alpha near 1 (long memory), an initial state, 4 segments
    of 48 tokens (three 16-token chunks each)."""
    from gdr_gen import make_gdn2
    _check2(gdr_lib, make_gdn2(B=1, T=192, H=3, Dk=dims[0], Dv=dims[1], dtype="bf16",
                               seed=800 + dims[0] + dims[1], alpha_shift=-4.0, s0_std=0.05),
            4, 30)


def test_gdr2_bwd_split_norm_ragged(gdr_lib):
    """q, k normalised on load, segments of 40 tokens (not a multiple of
    the chunk), two sequences."""
    from gdr_gen import make_gdn2
    _check2(gdr_lib, make_gdn2(B=2, T=200, H=2, Dk=128, Dv=128, dtype="bf16", seed=810,
                               alpha_shift=-3.0, s0_std=0.05, raw_qk=True), 5, 31, norm=True)
