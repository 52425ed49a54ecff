"""GPU parity of gdr_chunk_fwd_gate: the scalar-gate forward with the block's
output gate (RMSNorm x SiLU) fused on its stores.

Expected values are the oracle's composition on the same seeded inputs,
``rmsnorm_gate(gdn_fwd(q, k, v, alpha, beta, s0).o, g, w, eps)``, in fp64.
Metric: max error over rms(y) <= 2e-2 for bf16 inputs and 1e-3 for fp32
inputs (the forward's tolerances; the gate itself is fp32 arithmetic on the
forward's output), plus the measured bf16 rounding floor of the oracle's y
when y is bf16; the final state as for gdr_chunk_fwd.  Shapes cover one to
many row blocks per head (1, 2, 4 and 8 workgroups share a head's rows and
exchange per-token sums), ragged and single-chunk sequences, both head dims.
"""
import numpy as np
import pytest
import torch

import oracle
from gdr_gen import make_config, make_gate, make_gdn

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-3, "bf16": 2e-2}
DT = {"f32": torch.float32, "bf16": torch.bfloat16}


def _gpu(x):
    return None if x is None else x.cuda()


def _gate_inputs(B, T, H, Dv, g_dt, seed, weight=True):
    gi = make_gate(B * T, H, Dv, "f32", g_dt, seed=seed, weight=weight)
    return gi.g.reshape(B, T, H, Dv), gi.w


def _tol(in_dt, out_dt, y_ref):
    t = TOL[in_dt]
    if out_dt == "bf16":
        yb = torch.from_numpy(np.asarray(y_ref, dtype=np.float32)).to(torch.bfloat16)
        t += oracle.err_rms(yb.double().numpy(), y_ref)
    return t


def _check(gdr_lib, inp, g_dt="bf16", out="f32", eps=1e-6, weight=True, l2norm=False, seed=7):
    B, T, H, Dk = inp.q.shape
    Dv = inp.v.shape[-1]
    print(f"fused gate B{B} T{T} H{H} Dk{Dk} Dv{Dv} in={inp.dtype} g={g_dt} y={out} "
          f"eps={eps} w={weight} l2norm={l2norm}", flush=True)
    g, w = _gate_inputs(B, T, H, Dv, g_dt, seed, weight)
    q, k = inp.q, inp.k
    if l2norm:
        q, k = oracle.l2norm(q), oracle.l2norm(k)
    o_ref, s_ref = oracle.gdn_fwd(q, k, inp.v, inp.alpha, inp.beta, inp.s0)
    y_ref = oracle.rmsnorm_gate(o_ref, g, w, eps=eps)
    y, s = gdr_lib.gdr_chunk_fwd_gate(_gpu(inp.q), _gpu(inp.k), _gpu(inp.v), _gpu(inp.alpha),
                                      _gpu(inp.beta), _gpu(inp.s0), _gpu(g), _gpu(w), eps,
                                      out_dtype=DT[out], l2norm_qk=l2norm)
    torch.cuda.synchronize()
    ey, es = oracle.err_rms(y.cpu(), y_ref), oracle.err_rms(s.cpu(), s_ref)
    print(f"  err y {ey:.2e}  S {es:.2e}")
    assert ey <= _tol(inp.dtype, out, y_ref) and es <= TOL[inp.dtype], (ey, es)


@pytest.mark.parametrize("T", [1, 31, 32, 33, 65, 100])
def test_fused_gate_ragged_short(gdr_lib, T):
    # B1 H2 d128: narrow row blocks, eight workgroups per head
    _check(gdr_lib, make_gdn(B=1, T=T, H=2, Dk=128, Dv=128, dtype="bf16", seed=600 + T,
                             s0_std=0.05))


@pytest.mark.parametrize("Dk,Dv", [(64, 64), (64, 128), (128, 64), (128, 128)])
@pytest.mark.parametrize("B,H", [(1, 3), (8, 16)])
def test_fused_gate_head_dims(gdr_lib, Dk, Dv, B, H):
    # (1, 3): 16-row blocks (4 or 8 per head); (8, 16): 64-row blocks (1 or 2)
    _check(gdr_lib, make_gdn(B=B, T=130, H=H, Dk=Dk, Dv=Dv, dtype="bf16", seed=610 + Dk + Dv,
                             s0_std=0.05))


@pytest.mark.parametrize("g_dt,out", [("bf16", "bf16"), ("f32", "f32"), ("f32", "bf16")])
def test_fused_gate_dtypes(gdr_lib, g_dt, out):
    _check(gdr_lib, make_gdn(B=4, T=200, H=16, Dk=128, Dv=128, dtype="bf16", seed=620),
           g_dt=g_dt, out=out)


@pytest.mark.parametrize("eps,weight", [(0.0, True), (1e-2, False), (1.0, True)])
def test_fused_gate_eps_and_weight(gdr_lib, eps, weight):
    _check(gdr_lib, make_gdn(B=2, T=97, H=4, Dk=128, Dv=128, dtype="bf16", seed=630),
           eps=eps, weight=weight)


def test_fused_gate_with_l2norm(gdr_lib):
    _check(gdr_lib, make_gdn(B=4, T=160, H=16, Dk=128, Dv=128, dtype="bf16", seed=640,
                             raw_qk=True), l2norm=True)


@pytest.mark.parametrize("T", [1, 77])
def test_fused_gate_fp32_inputs(gdr_lib, T):
    # fp32 inputs: the vector-ALU forward into the workspace, then the gate
    _check(gdr_lib, make_gdn(B=2, T=T, H=3, Dk=64, Dv=128, dtype="f32", seed=650 + T,
                             s0_std=0.1), g_dt="f32")


def test_fused_gate_equals_two_calls(gdr_lib):
    """The fused call agrees with gdr_output_gate(gdr_chunk_fwd(...)) to fp32
    rounding: the same o from the same kernel code, the gate's operations in
    another order."""
    inp = make_gdn(B=8, T=300, H=16, Dk=128, Dv=128, dtype="bf16", seed=660, s0_std=0.05)
    g, w = _gate_inputs(8, 300, 16, 128, "bf16", 661)
    args = [_gpu(x) for x in (inp.q, inp.k, inp.v, inp.alpha, inp.beta, inp.s0)]
    o, s1 = gdr_lib.gdr_chunk_fwd(*args, out_dtype=torch.float32)
    y1 = gdr_lib.gdr_output_gate(o, _gpu(g), _gpu(w), 1e-6, out_dtype=torch.float32)
    y2, s2 = gdr_lib.gdr_chunk_fwd_gate(*args, _gpu(g), _gpu(w), 1e-6, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(s1, s2)
    rel = ((y1 - y2).abs().max() / y1.pow(2).mean().sqrt()).item()
    assert rel <= 1e-5, rel


def test_fused_gate_workload_b8_h16_t4096(gdr_lib):
    """The full B8 H16 T4096 d128 workload, y and the final state of every
    head against the oracle."""
    inp = make_config(1)
    B, T, H, Dk = inp.q.shape
    g, w = _gate_inputs(B, T, H, 128, "bf16", 670)
    y, s = gdr_lib.gdr_chunk_fwd_gate(*[_gpu(x) for x in (inp.q, inp.k, inp.v, inp.alpha,
                                                          inp.beta, inp.s0)],
                                      _gpu(g), _gpu(w), 1e-6, out_dtype=torch.float32)
    torch.cuda.synchronize()
    y, s = y.cpu(), s.cpu()
    for bi in range(B):
        sl = slice(bi, bi + 1)
        o_ref, s_ref = oracle.gdn_fwd(inp.q[sl], inp.k[sl], inp.v[sl], inp.alpha[sl],
                                      inp.beta[sl], None)
        y_ref = oracle.rmsnorm_gate(o_ref, g[sl], w, eps=1e-6)
        ey, es = oracle.err_rms(y[sl], y_ref), oracle.err_rms(s[sl], s_ref)
        print(f"  batch {bi}: err y {ey:.2e}  S {es:.2e}", flush=True)
        assert ey <= 2e-2 and es <= 2e-2, (bi, ey, es)


def test_fused_gate_empty_sequence_copies_state(gdr_lib):
    inp = make_gdn(B=2, T=1, H=2, Dk=64, Dv=64, dtype="bf16", seed=680, s0_std=0.1)
    q = inp.q[:, :0].contiguous()
    g = torch.zeros((2, 0, 2, 64), dtype=torch.bfloat16)
    y, s = gdr_lib.gdr_chunk_fwd_gate(_gpu(q), _gpu(q.clone()), _gpu(inp.v[:, :0].contiguous()),
                                      _gpu(inp.alpha[:, :0].contiguous()),
                                      _gpu(inp.beta[:, :0].contiguous()), _gpu(inp.s0), _gpu(g),
                                      None, 1e-6, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert y.numel() == 0 and torch.equal(s.cpu(), inp.s0)
