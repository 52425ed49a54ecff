"""GPU cross-path checks: the chunked kernel against the decode kernel, the
state hand-off across calls, special cases with closed forms, and run-to-run
determinism."""
import numpy as np
import pytest
import torch

import oracle
from gdr_gen import make_gdn

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _g(x):
    return None if x is None else x.to(DEV)


@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_chunk_equals_recurrent_steps(gdr_lib, dt):
    inp = make_gdn(B=2, T=70, H=2, Dk=128, Dv=128, dtype=dt, seed=21,
                   s0_std=0.05)
    o, s = gdr_lib.gdr_chunk_fwd(_g(inp.q), _g(inp.k), _g(inp.v),
                                 _g(inp.alpha), _g(inp.beta), _g(inp.s0),
                                 out_dtype=torch.float32)
    st = _g(inp.s0.clone())
    outs = []
    for t in range(70):
        outs.append(gdr_lib.gdr_recurrent_step(
            _g(inp.q[:, t].contiguous()), _g(inp.k[:, t].contiguous()),
            _g(inp.v[:, t].contiguous()), _g(inp.alpha[:, t].contiguous()),
            _g(inp.beta[:, t].contiguous()), st, out_dtype=torch.float32))
    o2 = torch.stack(outs, 1)
    torch.cuda.synchronize()
    tol = 2e-2 if dt == "bf16" else 1e-3
    assert oracle.err_rms(o2.cpu(), o.cpu()) <= tol
    assert oracle.err_rms(st.cpu(), s.cpu()) <= tol


@pytest.mark.parametrize("T1", [1, 50, 64, 100])
def test_split_invariance(gdr_lib, T1):
    """run(T) == run(T1) then run(T - T1) from the handed-over state."""
    inp = make_gdn(B=1, T=200, H=2, Dk=128, Dv=128, dtype="bf16", seed=22,
                   s0_std=0.05)
    q, k, v, a, b = map(_g, (inp.q, inp.k, inp.v, inp.alpha, inp.beta))
    o, s = gdr_lib.gdr_chunk_fwd(q, k, v, a, b, _g(inp.s0),
                                 out_dtype=torch.float32)
    sl = lambda x, lo, hi: x[:, lo:hi].contiguous()  # noqa: E731
    oa, sa = gdr_lib.gdr_chunk_fwd(sl(q, 0, T1), sl(k, 0, T1), sl(v, 0, T1),
                                   sl(a, 0, T1), sl(b, 0, T1), _g(inp.s0),
                                   out_dtype=torch.float32)
    ob, sb = gdr_lib.gdr_chunk_fwd(sl(q, T1, 200), sl(k, T1, 200),
                                   sl(v, T1, 200), sl(a, T1, 200),
                                   sl(b, T1, 200), sa, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert oracle.err_rms(torch.cat([oa, ob], 1).cpu(), o.cpu()) <= 2e-2
    assert oracle.err_rms(sb.cpu(), s.cpu()) <= 2e-2


def test_pure_decay_closed_form(gdr_lib):
    """beta = 0: S_t = (prod alpha) S_0 and o_t = (prod_{i<=t} alpha_i) S_0 q_t
    across 512 chunks (closed form, fp64 log-space products)."""
    inp = make_gdn(B=1, T=32768, H=4, Dk=128, Dv=128, dtype="bf16", seed=23,
                   s0_std=0.02, alpha_shift=-7.0)
    beta = torch.zeros_like(inp.beta)
    o, s = gdr_lib.gdr_chunk_fwd(_g(inp.q), _g(inp.k), _g(inp.v),
                                 _g(inp.alpha), _g(beta), _g(inp.s0),
                                 out_dtype=torch.float32)
    torch.cuda.synchronize()
    cum = np.exp(np.cumsum(np.log(inp.alpha.double().numpy()), axis=1))
    S0 = inp.s0.double().numpy()
    q = inp.q.double().numpy()
    ref_o = np.einsum("bth,bhij,bthj->bthi", cum, S0, q)
    ref_s = cum[:, -1][:, :, None, None] * S0
    assert oracle.err_rms(o.cpu(), ref_o) <= 2e-2
    assert oracle.err_rms(s.cpu(), ref_s) <= 2e-2


def test_alpha_zero_is_reset(gdr_lib):
    """alpha = 0 forgets everything before the token, without NaN."""
    inp = make_gdn(B=1, T=130, H=2, Dk=128, Dv=128, dtype="bf16", seed=24,
                   s0_std=0.05)
    a = inp.alpha.clone()
    a[:, 70] = 0.0
    o, s = gdr_lib.gdr_chunk_fwd(_g(inp.q), _g(inp.k), _g(inp.v), _g(a),
                                 _g(inp.beta), _g(inp.s0),
                                 out_dtype=torch.float32)
    o_ref, s_ref = oracle.gdn_fwd(inp.q, inp.k, inp.v, a, inp.beta, inp.s0)
    torch.cuda.synchronize()
    assert torch.isfinite(o).all() and torch.isfinite(s).all()
    assert oracle.err_rms(o.cpu(), o_ref) <= 2e-2
    assert oracle.err_rms(s.cpu(), s_ref) <= 2e-2


def test_deterministic(gdr_lib):
    inp = make_gdn(B=2, T=300, H=4, Dk=128, Dv=128, dtype="bf16", seed=25,
                   s0_std=0.05)
    args = [_g(x) for x in (inp.q, inp.k, inp.v, inp.alpha, inp.beta,
                            inp.s0)]
    o1, s1 = gdr_lib.gdr_chunk_fwd(*args, out_dtype=torch.float32)
    o2, s2 = gdr_lib.gdr_chunk_fwd(*args, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(s1, s2)


def test_empty_sequence_copies_state(gdr_lib):
    s0 = torch.randn(2, 3, 64, 64, device=DEV)
    e = torch.empty(2, 0, 3, 64, device=DEV, dtype=torch.bfloat16)
    a = torch.empty(2, 0, 3, device=DEV)
    o, s = gdr_lib.gdr_chunk_fwd(e, e, e, a, a, s0)
    torch.cuda.synchronize()
    assert o.shape == (2, 0, 3, 64) and torch.equal(s, s0)


def test_gdn2_collapses_to_gdn(gdr_lib):
    """Gated Delta Rule-2 with every gate collapsed to one scalar per token
    (alpha, b = w = beta on all channels) is the scalar gated rule: the two
    kernels agree.  Gates are bf16-exact so both see the same values."""
    inp = make_gdn(B=2, T=150, H=2, Dk=128, Dv=128, dtype="bf16", seed=26,
                   s0_std=0.05)
    a = inp.alpha.to(torch.bfloat16)
    b = inp.beta.to(torch.bfloat16)
    Dk, Dv = 128, 128
    o1, s1 = gdr_lib.gdr_chunk_fwd(_g(inp.q), _g(inp.k), _g(inp.v),
                                   _g(a.float()), _g(b.float()), _g(inp.s0),
                                   out_dtype=torch.float32)
    o2, s2 = gdr_lib.gdr2_chunk_fwd(
        _g(inp.q), _g(inp.k), _g(inp.v),
        _g(a[..., None].expand(-1, -1, -1, Dk).contiguous()),
        _g(b[..., None].expand(-1, -1, -1, Dk).contiguous()),
        _g(b[..., None].expand(-1, -1, -1, Dv).contiguous()), _g(inp.s0),
        out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert oracle.err_rms(o2.cpu(), o1.cpu()) <= 2e-2
    assert oracle.err_rms(s2.cpu(), s1.cpu()) <= 2e-2


def test_gdn2_kda_collapse(gdr_lib):
    """b = w = beta (per token) with per-channel alpha: the KDA special case
    against the oracle."""
    from gdr_gen import make_gdn2
    inp = make_gdn2(B=1, T=130, H=2, Dk=128, Dv=128, dtype="bf16", seed=27,
                    s0_std=0.05)
    beta = inp.erase[..., :1]
    e = beta.expand(-1, -1, -1, 128).contiguous()
    w = beta.expand(-1, -1, -1, 128).contiguous()
    o, s = gdr_lib.gdr2_chunk_fwd(_g(inp.q), _g(inp.k), _g(inp.v),
                                  _g(inp.alpha), _g(e), _g(w), _g(inp.s0),
                                  out_dtype=torch.float32)
    o_ref, s_ref = oracle.gdn2_fwd(inp.q, inp.k, inp.v, inp.alpha, e, w,
                                   inp.s0)
    torch.cuda.synchronize()
    assert oracle.err_rms(o.cpu(), o_ref) <= 2e-2
    assert oracle.err_rms(s.cpu(), s_ref) <= 2e-2
