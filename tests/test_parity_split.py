"""GPU parity of gdr_chunk_fwd_split (each sequence split into segments that
run side by side, composed through their affine state maps) against the fp64
oracle's token-by-token recurrence, on o and the final state, at the
tolerances of the plain call: 2e-2 of rms for bf16 inputs, 1e-3 for fp32."""
import pytest
import torch

import oracle
from gdr_gen import make_config, make_gdn

pytestmark = pytest.mark.gpu

TOL = {"bf16": 2e-2, "f32": 1e-3}


def _gpu(x):
    return None if x is None else x.cuda()


def _check(gdr_lib, inp, nseg, odt=torch.float32, l2norm=False, tol=None):
    print(f"split nseg={nseg} {inp.meta} out={odt} l2norm={l2norm}", flush=True)
    qn, kn = inp.q, inp.k
    if l2norm:
        qn = torch.from_numpy(oracle.l2norm(inp.q))
        kn = torch.from_numpy(oracle.l2norm(inp.k))
    o_ref, s_ref = oracle.gdn_fwd(qn, kn, inp.v, inp.alpha, inp.beta, inp.s0)
    o, s = gdr_lib.gdr_chunk_fwd_split(_gpu(inp.q), _gpu(inp.k), _gpu(inp.v), _gpu(inp.alpha),
                                       _gpu(inp.beta), _gpu(inp.s0), nseg=nseg, out_dtype=odt,
                                       l2norm_qk=l2norm)
    torch.cuda.synchronize()
    eo, es = oracle.err_rms(o.cpu(), o_ref), oracle.err_rms(s.cpu(), s_ref)
    tol = TOL[inp.dtype] if tol is None else tol
    print(f"  err(o)={eo:.3e} err(S)={es:.3e} tol={tol}")
    assert eo <= tol and es <= tol, (eo, es)


@pytest.mark.parametrize("nseg", [2, 4, 8])
def test_split_bf16_long_memory(gdr_lib, nseg):
    """alpha near 1: the segment transitions P carry most of the state."""
    _check(gdr_lib, make_gdn(B=1, T=512, H=2, Dk=128, Dv=128, dtype="bf16", seed=700 + nseg,
                             alpha_shift=-4.0, s0_std=0.05), nseg)


@pytest.mark.parametrize("nseg", [2, 5])
def test_split_bf16_fast_decay_ragged_segments(gdr_lib, nseg):
    """Segments of 90 and 36 tokens: not multiples of the chunk."""
    _check(gdr_lib, make_gdn(B=2, T=180, H=2, Dk=128, Dv=128, dtype="bf16", seed=710 + nseg,
                             s0_std=0.05), nseg)


@pytest.mark.parametrize("dims", [(128, 64), (64, 128), (64, 64)])
def test_split_bf16_dims(gdr_lib, dims):
    """Dk != Dv: the P pass has its own d_k x d_k state and output."""
    _check(gdr_lib, make_gdn(B=1, T=256, H=3, Dk=dims[0], Dv=dims[1], dtype="bf16",
                             seed=720 + dims[0] + dims[1], alpha_shift=-2.0, s0_std=0.1), 4)


@pytest.mark.parametrize("dims", [(64, 64), (128, 64), (64, 128)])
def test_split_f32(gdr_lib, dims):
    """fp32 inputs run the vector-ALU chunk kernel in every pass; with
    Dk != Dv its P pass writes the workspace's bf16 buffer."""
    _check(gdr_lib, make_gdn(B=1, T=256, H=2, Dk=dims[0], Dv=dims[1], dtype="f32",
                             seed=730 + (dims != (64, 64)) * (dims[0] + 2 * dims[1]),
                             alpha_shift=-3.0, s0_std=0.2), 4)


def test_split_bf16_out_and_l2norm(gdr_lib):
    """bf16 output, and q, k normalised on load in all three passes."""
    inp = make_gdn(B=1, T=256, H=2, Dk=128, Dv=128, dtype="bf16", seed=740, alpha_shift=-3.0,
                   s0_std=0.05, raw_qk=True)
    _check(gdr_lib, inp, 4, odt=torch.bfloat16, l2norm=True)


def test_split_one_segment_is_plain(gdr_lib):
    """nseg = 1 is the plain call: identical results."""
    inp = make_gdn(B=1, T=100, H=2, Dk=128, Dv=128, dtype="bf16", seed=750, s0_std=0.05)
    args = [_gpu(x) for x in (inp.q, inp.k, inp.v, inp.alpha, inp.beta, inp.s0)]
    o1, s1 = gdr_lib.gdr_chunk_fwd(*args, out_dtype=torch.float32)
    o2, s2 = gdr_lib.gdr_chunk_fwd_split(*args, nseg=1, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(s1, s2)


def test_split_long_context_workload(gdr_lib):
    """The long-context workload, B1 H16 T32768 d128 with a random initial
    state and alpha near 1, in 8 segments of 4096 tokens (the launch the
    benchmark times)."""
    _check(gdr_lib, make_config(2), 8)
