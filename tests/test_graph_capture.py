"""The C-ABI calls under HIP graph capture (torch.cuda.CUDAGraph on the
capturing stream): every call enqueues kernels only (no memset nodes, no
allocation, no host synchronisation), so a captured sequence replays to the
same bits as the eager calls -- but for the backwards' gradients that are
summed over blocks of state rows by atomic adds (dq, dk, and GDN-2's dalpha
and derase), whose order varies: those match to fp32 rounding.  Each replay
is separated by eager work and a synchronisation, and every replay is
checked."""
import pytest
import torch

from gdr_gen import make_decode, make_gdn, make_gdn2

pytestmark = pytest.mark.gpu


def _replays_match(fn, outs_eager, n=3, summed=()):
    """summed: indices of outputs that atomic adds produce"""
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()                      # warm-up on the capture stream (attribute setup)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        outs = fn()
    for i in range(n):
        junk = torch.randn(1 << 20, device="cuda").sum()   # eager work between replays
        torch.cuda.synchronize()
        for o in outs:
            o.zero_()
        g.replay()
        torch.cuda.synchronize()
        for j, (a, b) in enumerate(zip(outs, outs_eager)):
            if j in summed:
                assert ((a - b).abs().max() <= 1e-5 * b.abs().max()).item(), \
                    f"replay {i} output {j} differs"
            else:
                assert torch.equal(a, b), f"replay {i} output {j} differs"
        del junk


def test_graph_chunk_fwd_and_decode(gdr_lib):
    inp = make_gdn(B=2, T=100, H=2, Dk=128, Dv=128, dtype="bf16", seed=900, s0_std=0.05)
    args = [x.cuda() for x in (inp.q, inp.k, inp.v, inp.alpha, inp.beta, inp.s0)]
    dec = make_decode(N=4, H=2, Dk=128, Dv=128, steps=1, dtype="bf16", seed=901)
    dargs = [x[0].cuda() for x in (dec.q, dec.k, dec.v, dec.alpha, dec.beta)]
    st0 = dec.state0.cuda()
    o = torch.empty((2, 100, 2, 128), dtype=torch.float32, device="cuda")
    sf = torch.empty((2, 2, 128, 128), dtype=torch.float32, device="cuda")
    od = torch.empty((4, 2, 128), dtype=torch.float32, device="cuda")
    st = torch.empty_like(st0)

    def fn():
        gdr_lib.gdr_chunk_fwd(*args, out_dtype=torch.float32, o=o, s_final=sf)
        st.copy_(st0)
        gdr_lib.gdr_recurrent_step(*dargs, st, out_dtype=torch.float32, o=od)
        return o, sf, od, st

    fn()
    torch.cuda.synchronize()
    eager = [x.clone() for x in (o, sf, od, st)]
    _replays_match(fn, eager)


def test_graph_gdr2_and_backward(gdr_lib):
    inp = make_gdn2(B=1, T=70, H=2, Dk=128, Dv=128, dtype="bf16", seed=902, s0_std=0.05)
    args = [x.cuda() for x in (inp.q, inp.k, inp.v, inp.alpha, inp.erase, inp.write, inp.s0)]
    o = torch.empty((1, 70, 2, 128), dtype=torch.float32, device="cuda")
    sf = torch.empty((1, 2, 128, 128), dtype=torch.float32, device="cuda")
    do = torch.randn((1, 70, 2, 128), device="cuda")
    ws = torch.empty(gdr_lib.gdr2_chunk_bwd_workspace_size(1, 70, 2, 128, 128),
                     dtype=torch.uint8, device="cuda")
    grads = {}

    def fn():
        gdr_lib.gdr2_chunk_fwd(*args, out_dtype=torch.float32, o=o, s_final=sf)
        g = gdr_lib.gdr2_chunk_bwd(*args, do, None, workspace=ws)
        grads["g"] = g
        return (o, sf) + tuple(g)

    outs = fn()
    torch.cuda.synchronize()
    eager = [x.clone() for x in outs]
    # (o, sf, dq, dk, dv, dalpha, derase, dwrite, ds0)
    _replays_match(fn, eager, summed=(2, 3, 5, 6))


def test_graph_split_forward(gdr_lib):
    inp = make_gdn(B=1, T=256, H=2, Dk=128, Dv=128, dtype="bf16", seed=903, alpha_shift=-3.0,
                   s0_std=0.05)
    args = [x.cuda() for x in (inp.q, inp.k, inp.v, inp.alpha, inp.beta, inp.s0)]
    o = torch.empty((1, 256, 2, 128), dtype=torch.float32, device="cuda")
    sf = torch.empty((1, 2, 128, 128), dtype=torch.float32, device="cuda")
    ws = torch.empty(gdr_lib.gdr_chunk_fwd_split_workspace_size(1, 256, 2, 128, 128,
                                                                torch.bfloat16, 4),
                     dtype=torch.uint8, device="cuda")

    def fn():
        gdr_lib.gdr_chunk_fwd_split(*args, nseg=4, out_dtype=torch.float32, o=o, s_final=sf,
                                    workspace=ws)
        return o, sf

    fn()
    torch.cuda.synchronize()
    eager = [x.clone() for x in (o, sf)]
    _replays_match(fn, eager)


def test_graph_split_backward_and_gate(gdr_lib):
    """The sequence-split backward (identity and zero fills are kernels),
    then the output gate and its reverse mode with the dw reduction."""
    from gdr_gen import make_gate
    inp = make_gdn(B=1, T=128, H=2, Dk=64, Dv=64, dtype="bf16", seed=904, alpha_shift=-2.0,
                   s0_std=0.05)
    args = [x.cuda() for x in (inp.q, inp.k, inp.v, inp.alpha, inp.beta, inp.s0)]
    do = torch.randn((1, 128, 2, 64), device="cuda")
    dsf = 0.1 * torch.randn((1, 2, 64, 64), device="cuda")
    ws = torch.empty(gdr_lib.gdr_chunk_bwd_split_workspace_size(1, 128, 2, 64, 64,
                                                                torch.bfloat16, 4),
                     dtype=torch.uint8, device="cuda")
    gi = make_gate(64, 2, 128, "f32", "bf16", seed=905)
    o, g, w = gi.o.cuda(), gi.g.cuda(), gi.w.cuda()
    dy = torch.randn(o.shape, device="cuda").to(torch.bfloat16)
    gws = torch.empty(gdr_lib.gdr_output_gate_bwd_workspace_size(64, 2, 128), dtype=torch.uint8,
                      device="cuda")

    def fn():
        grads = gdr_lib.gdr_chunk_bwd_split(*args, do, dsf, nseg=4, workspace=ws)
        y = gdr_lib.gdr_output_gate(o, g, w, 1e-6, out_dtype=torch.float32)
        gb = gdr_lib.gdr_output_gate_bwd(o, g, w, dy, 1e-6, workspace=gws)
        return tuple(grads) + (y,) + tuple(gb)

    outs = fn()
    torch.cuda.synchronize()
    eager = [x.clone() for x in outs]
    # (dq, dk, dv, dalpha, dbeta, ds0, y, ...)
    _replays_match(fn, eager, summed=(0, 1))
