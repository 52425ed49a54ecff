"""GPU parity of the fused L2 normalisation of q and k (GDR_L2NORM_QK).

The kernels receive raw q, k (per-token scales spread over [0.05, 20]) and
normalise them on load; the oracle runs the plain rule on
``oracle.l2norm(q)``, ``oracle.l2norm(k)`` (fp64, eps = 1e-6 inside the
root).  Same metric and tolerances as the other parity tests: max error over
rms(x) <= 1e-3 for fp32 inputs and 2e-2 for bf16 inputs, on o and on S.
"""
import ctypes

import numpy as np
import pytest
import torch

import oracle
from gdr_gen import make_decode, make_gdn, make_gdn2

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-3, "bf16": 2e-2}
DEV = "cuda"
EPS = 1e-6


def _n(x):
    return oracle.l2norm(x, eps=EPS)


def _gpu(x):
    return None if x is None else x.to(DEV)


def _odt(name):
    return torch.bfloat16 if name == "bf16" else torch.float32


def _tol(in_dt, out_dt, o_ref):
    t = TOL[in_dt]
    if out_dt == "bf16":
        xb = torch.from_numpy(np.asarray(o_ref, dtype=np.float32)).to(torch.bfloat16)
        t += oracle.err_rms(xb.double().numpy(), o_ref)
    return t


def _check_gdn(gdr_lib, inp, odt="f32"):
    print(f"GDN l2norm {inp.meta}", flush=True)
    o_ref, s_ref = oracle.gdn_fwd(_n(inp.q), _n(inp.k), inp.v, inp.alpha, inp.beta, inp.s0)
    o, s = gdr_lib.gdr_chunk_fwd(_gpu(inp.q), _gpu(inp.k), _gpu(inp.v), _gpu(inp.alpha),
                                 _gpu(inp.beta), _gpu(inp.s0), out_dtype=_odt(odt),
                                 l2norm_qk=True)
    torch.cuda.synchronize()
    eo, es = oracle.err_rms(o.cpu(), o_ref), oracle.err_rms(s.cpu(), s_ref)
    assert eo <= _tol(inp.dtype, odt, o_ref) and es <= TOL[inp.dtype], (eo, es)
    return eo, es


def _check_gdn2(gdr_lib, inp, odt="f32"):
    print(f"GDN-2 l2norm {inp.meta}", flush=True)
    o_ref, s_ref = oracle.gdn2_fwd(_n(inp.q), _n(inp.k), inp.v, inp.alpha, inp.erase,
                                   inp.write, inp.s0)
    o, s = gdr_lib.gdr2_chunk_fwd(_gpu(inp.q), _gpu(inp.k), _gpu(inp.v), _gpu(inp.alpha),
                                  _gpu(inp.erase), _gpu(inp.write), _gpu(inp.s0),
                                  out_dtype=_odt(odt), l2norm_qk=True)
    torch.cuda.synchronize()
    eo, es = oracle.err_rms(o.cpu(), o_ref), oracle.err_rms(s.cpu(), s_ref)
    assert eo <= _tol(inp.dtype, odt, o_ref) and es <= TOL[inp.dtype], (eo, es)
    return eo, es


# ------------------------------------------------------- scalar-gate rule ----

@pytest.mark.parametrize("T", [1, 33, 100, 257])
def test_gdn_bf16_l2norm_ragged(gdr_lib, T):
    _check_gdn(gdr_lib, make_gdn(B=1, T=T, H=2, Dk=128, Dv=128, dtype="bf16", seed=200 + T,
                                 s0_std=0.05, raw_qk=True))


@pytest.mark.parametrize("dims", [(128, 128), (128, 64), (64, 128), (64, 64)])
@pytest.mark.parametrize("odt", ["f32", "bf16"])
def test_gdn_bf16_l2norm_dims(gdr_lib, dims, odt):
    _check_gdn(gdr_lib, make_gdn(B=1, T=130, H=3, Dk=dims[0], Dv=dims[1], dtype="bf16",
                                 seed=210 + dims[0] + dims[1], s0_std=0.05, raw_qk=True), odt)


@pytest.mark.parametrize("dims", [(128, 128), (64, 64)])
def test_gdn_bf16_l2norm_many_heads(gdr_lib, dims):
    """Enough heads for the 64-row blocks (the launch shape of the large
    workloads)."""
    _check_gdn(gdr_lib, make_gdn(B=4, T=100, H=16, Dk=dims[0], Dv=dims[1], dtype="bf16",
                                 seed=220, s0_std=0.05, raw_qk=True))


@pytest.mark.parametrize("T", [1, 65, 130])
@pytest.mark.parametrize("dims", [(64, 64), (128, 128)])
def test_gdn_fp32_l2norm(gdr_lib, T, dims):
    _check_gdn(gdr_lib, make_gdn(B=1, T=T, H=2, Dk=dims[0], Dv=dims[1], dtype="f32",
                                 seed=230 + T, s0_std=0.5, raw_qk=True))


@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_gdn_l2norm_zero_rows(gdr_lib, dt):
    """A zero q or k row normalises to zero (eps keeps it finite): that
    token reads nothing from the state and writes nothing into it."""
    inp = make_gdn(B=1, T=90, H=2, Dk=128, Dv=128, dtype=dt, seed=240, s0_std=0.05,
                   raw_qk=True)
    q, k = inp.q.clone(), inp.k.clone()
    q[0, 5, 0] = 0
    q[0, 40:45, 1] = 0
    k[0, 6, 0] = 0
    k[0, 31:34, 1] = 0
    k[0, 89, 0] = 0
    inp.q, inp.k = q, k
    _check_gdn(gdr_lib, inp)


def test_gdn_bf16_l2norm_workload_b8_h16_t4096(gdr_lib):
    """The scalar-gate workload (B8 H16 T4096 d128 bf16) with raw q, k and
    the fused normalisation; the oracle checks batches 0 and 7."""
    inp = make_gdn(B=8, T=4096, H=16, Dk=128, Dv=128, dtype="bf16", seed=1001, raw_qk=True)
    print("GDN l2norm B8 H16 T4096", flush=True)
    o, s = gdr_lib.gdr_chunk_fwd(_gpu(inp.q), _gpu(inp.k), _gpu(inp.v), _gpu(inp.alpha),
                                 _gpu(inp.beta), None, out_dtype=torch.float32,
                                 l2norm_qk=True)
    torch.cuda.synchronize()
    o, s = o.cpu(), s.cpu()
    pick = [0, 7]
    o_ref, s_ref = oracle.gdn_fwd(_n(inp.q[pick]), _n(inp.k[pick]), inp.v[pick],
                                  inp.alpha[pick], inp.beta[pick], None)
    eo, es = oracle.err_rms(o[pick], o_ref), oracle.err_rms(s[pick], s_ref)
    print(f"err(o)={eo:.3e} err(S)={es:.3e}")
    assert eo <= TOL["bf16"] and es <= TOL["bf16"], (eo, es)


# ------------------------------------------------------ channel-gate rule ----

@pytest.mark.parametrize("T", [1, 17, 150])
def test_gdn2_bf16_l2norm_ragged(gdr_lib, T):
    _check_gdn2(gdr_lib, make_gdn2(B=1, T=T, H=2, Dk=128, Dv=128, dtype="bf16",
                                   seed=250 + T, s0_std=0.05, raw_qk=True))


@pytest.mark.parametrize("dims", [(128, 128), (128, 64), (64, 128), (64, 64)])
@pytest.mark.parametrize("odt", ["f32", "bf16"])
def test_gdn2_bf16_l2norm_dims(gdr_lib, dims, odt):
    _check_gdn2(gdr_lib, make_gdn2(B=1, T=100, H=3, Dk=dims[0], Dv=dims[1], dtype="bf16",
                                   seed=260 + dims[0] + dims[1], s0_std=0.05, raw_qk=True),
                odt)


@pytest.mark.parametrize("dims", [(128, 128), (64, 64)])
def test_gdn2_bf16_l2norm_wide_decay_range(gdr_lib, dims):
    """Blocks whose channel decay passes the factored form's limit take the
    entry-by-entry path, which reads the raw q, k and applies the norms
    there."""
    inp = make_gdn2(B=1, T=140, H=2, Dk=dims[0], Dv=dims[1], dtype="bf16", seed=270,
                    s0_std=0.05, raw_qk=True)
    a = inp.alpha.clone()
    a[0, 20:23, 0, 5] = 1e-12
    a[0, 70, 1, :] = 0.0
    a[0, 100:116, 1, 7] = 0.004
    inp.alpha = a
    _check_gdn2(gdr_lib, inp)


@pytest.mark.parametrize("T", [1, 70])
def test_gdn2_fp32_l2norm(gdr_lib, T):
    _check_gdn2(gdr_lib, make_gdn2(B=1, T=T, H=2, Dk=64, Dv=128, dtype="f32", seed=280 + T,
                                   s0_std=0.5, raw_qk=True))


def test_gdn2_bf16_l2norm_zero_rows(gdr_lib):
    inp = make_gdn2(B=1, T=60, H=2, Dk=128, Dv=128, dtype="bf16", seed=290, s0_std=0.05,
                    raw_qk=True)
    q, k = inp.q.clone(), inp.k.clone()
    q[0, 3, 0] = 0
    k[0, 16:18, 1] = 0
    k[0, 59, 0] = 0
    inp.q, inp.k = q, k
    _check_gdn2(gdr_lib, inp)


# ------------------------------------------------------------------ decode ----

@pytest.mark.parametrize("dims", [(128, 128), (64, 64), (128, 64), (64, 128)])
@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_step_l2norm(gdr_lib, dims, dt):
    dec = make_decode(N=8, H=4, Dk=dims[0], Dv=dims[1], steps=3, dtype=dt, seed=300,
                      raw_qk=True)
    print(f"step l2norm {dec.meta}", flush=True)
    st_ref = dec.state0.double().numpy().copy()
    st = _gpu(dec.state0.clone())
    for t in range(3):
        o_ref = oracle.gdn_step(_n(dec.q[t]), _n(dec.k[t]), dec.v[t], dec.alpha[t],
                                dec.beta[t], st_ref)
        o = gdr_lib.gdr_recurrent_step(_gpu(dec.q[t]), _gpu(dec.k[t]), _gpu(dec.v[t]),
                                       _gpu(dec.alpha[t]), _gpu(dec.beta[t]), st,
                                       out_dtype=torch.float32, l2norm_qk=True)
        torch.cuda.synchronize()
        eo = oracle.err_rms(o.cpu(), o_ref)
        es = oracle.err_rms(st.cpu(), st_ref)
        assert eo <= TOL[dt] and es <= TOL[dt], (t, eo, es)


# ---------------------------------------------------------- flags == 0 ----

def test_ex_with_no_flags_is_the_plain_call(gdr_lib):
    """The _ex entry points with flags = 0 give the plain calls' bits."""
    lib = gdr_lib.lib
    inp = make_gdn(B=2, T=77, H=3, Dk=128, Dv=128, dtype="bf16", seed=310, s0_std=0.05)
    args = [_gpu(x) for x in (inp.q, inp.k, inp.v, inp.alpha, inp.beta, inp.s0)]
    o1, s1 = gdr_lib.gdr_chunk_fwd(*args)
    o2 = torch.empty_like(o1)
    s2 = torch.empty_like(s1)
    p = lambda t: ctypes.c_void_p(t.data_ptr())
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    rc = lib.gdr_chunk_fwd_ex(2, 77, 3, 128, 128, 1, *[p(a) for a in args], 1, p(o2), p(s2),
                              0, st)
    torch.cuda.synchronize()
    assert rc == 0
    assert torch.equal(o1, o2) and torch.equal(s1, s2)

    inp = make_gdn2(B=1, T=50, H=2, Dk=128, Dv=128, dtype="bf16", seed=311, s0_std=0.05)
    args = [_gpu(x) for x in (inp.q, inp.k, inp.v, inp.alpha, inp.erase, inp.write, inp.s0)]
    o1, s1 = gdr_lib.gdr2_chunk_fwd(*args)
    o2 = torch.empty_like(o1)
    s2 = torch.empty_like(s1)
    rc = lib.gdr2_chunk_fwd_ex(1, 50, 2, 128, 128, 1, *[p(a) for a in args], 1, p(o2), p(s2),
                               0, st)
    torch.cuda.synchronize()
    assert rc == 0
    assert torch.equal(o1, o2) and torch.equal(s1, s2)
