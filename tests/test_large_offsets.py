"""Maximum sizes: tensors whose flat element offsets pass 2^31, so that any
32-bit index arithmetic would land on the wrong head, token or row.

Inputs are drawn in device memory by ``gdr_gen.make_device`` (a host draw of
this many values would take minutes).  Each call runs once over the whole
tensor, then sampled heads (or rows) -- always including the last one in the
buffer and ones at the far end of the batch -- are copied to the host
and checked against the fp64 oracle on those same bits, at the call's
tolerance (2e-2 of rms for bf16 inputs, 1e-3 for the fp32 output gate).
The backward is not run at this size: its workspace (chunk states and
partial sums) would exceed 140 GB, and its kernels address every tensor
with 64-bit offsets."""
import pytest
import torch

import oracle
from gdr_gen import make_device

pytestmark = pytest.mark.gpu

BF = torch.bfloat16
F32 = torch.float32
# B T H d: q, k, v and o hold 512 * 264 * 128 * 128 = 2.21e9 elements each
B, T, H, D = 512, 264, 128, 128
HEADS = [(0, 0), (0, H - 1), (B // 2, 64), (400, 99), (B - 1, 0), (B - 1, H - 1)]


def _err(x, ref):
    return oracle.err_rms(x.double().numpy(), ref)


def test_chunk_fwd_past_2_31_elements(gdr_lib):
    assert B * T * H * D > 2 ** 31
    print(f"gdr_chunk_fwd B{B} T{T} H{H} d{D}", flush=True)
    x = make_device({"q": ((B, T, H, D), "unit", BF), "k": ((B, T, H, D), "unit", BF),
                     "v": ((B, T, H, D), "normal", BF), "alpha": ((B, T, H), "decay", F32),
                     "beta": ((B, T, H), "gate", F32)}, seed=5100)
    o, sf = gdr_lib.gdr_chunk_fwd(x["q"], x["k"], x["v"], x["alpha"], x["beta"], None,
                                  out_dtype=F32)
    torch.cuda.synchronize()
    for b, h in HEADS:
        sl = (slice(b, b + 1), slice(None), slice(h, h + 1))
        o_ref, s_ref = oracle.gdn_fwd(*(x[n][sl].cpu() for n in ("q", "k", "v", "alpha", "beta")),
                                      None)
        eo, es = _err(o[sl].cpu(), o_ref), _err(sf[b:b + 1, h:h + 1].cpu(), s_ref)
        print(f"  head ({b}, {h}): err(o)={eo:.2e} err(S)={es:.2e}")
        assert eo <= 2e-2 and es <= 2e-2, (b, h, eo, es)


def test_gdr2_chunk_fwd_past_2_31_elements(gdr_lib):
    print(f"gdr2_chunk_fwd B{B} T{T} H{H} d{D}", flush=True)
    names = ("q", "k", "v", "alpha", "erase", "write")
    x = make_device({"q": ((B, T, H, D), "unit", BF), "k": ((B, T, H, D), "unit", BF),
                     "v": ((B, T, H, D), "normal", BF), "alpha": ((B, T, H, D), "decay", BF),
                     "erase": ((B, T, H, D), "gate", BF), "write": ((B, T, H, D), "gate", BF)},
                    seed=5200)
    o, sf = gdr_lib.gdr2_chunk_fwd(*(x[n] for n in names), None, out_dtype=F32)
    torch.cuda.synchronize()
    for b, h in HEADS:
        sl = (slice(b, b + 1), slice(None), slice(h, h + 1))
        o_ref, s_ref = oracle.gdn2_fwd(*(x[n][sl].cpu() for n in names), None)
        eo, es = _err(o[sl].cpu(), o_ref), _err(sf[b:b + 1, h:h + 1].cpu(), s_ref)
        print(f"  head ({b}, {h}): err(o)={eo:.2e} err(S)={es:.2e}")
        assert eo <= 2e-2 and es <= 2e-2, (b, h, eo, es)


def test_decode_state_past_2_31_elements(gdr_lib):
    N, Hd = 2049, 64
    assert N * Hd * D * D > 2 ** 31
    print(f"gdr_recurrent_step N{N} H{Hd} d{D}", flush=True)
    x = make_device({"q": ((N, Hd, D), "unit", BF), "k": ((N, Hd, D), "unit", BF),
                     "v": ((N, Hd, D), "normal", BF), "alpha": ((N, Hd), "decay", F32),
                     "beta": ((N, Hd), "gate", F32), "state": ((N, Hd, D, D), "normal", F32)},
                    seed=5300)
    st = x["state"].mul_(0.02)
    heads = [(0, 0), (N // 2, 33), (N - 1, 0), (N - 1, Hd - 1)]
    before = {nh: st[nh[0]:nh[0] + 1, nh[1]:nh[1] + 1].cpu().double().numpy().copy()
              for nh in heads}
    o = gdr_lib.gdr_recurrent_step(x["q"], x["k"], x["v"], x["alpha"], x["beta"], st,
                                   out_dtype=F32)
    torch.cuda.synchronize()
    for (n, h) in heads:
        sl = (slice(n, n + 1), slice(h, h + 1))
        s_ref = before[(n, h)]
        o_ref = oracle.gdn_step(*(x[k][sl].cpu() for k in ("q", "k", "v", "alpha", "beta")),
                                s_ref)
        eo, es = _err(o[sl].cpu(), o_ref), _err(st[sl].cpu(), s_ref)
        print(f"  head ({n}, {h}): err(o)={eo:.2e} err(S)={es:.2e}")
        assert eo <= 2e-2 and es <= 2e-2, (n, h, eo, es)


def test_output_gate_past_2_31_elements(gdr_lib):
    N, Hg = 131073, 128
    assert N * Hg * D > 2 ** 31
    print(f"gdr_output_gate N{N} H{Hg} d{D}", flush=True)
    x = make_device({"o": ((N, Hg, D), "normal", F32), "g": ((N, Hg, D), "normal", BF),
                     "w": ((1, D), "gate", F32)}, seed=5400)
    y = gdr_lib.gdr_output_gate(x["o"], x["g"], x["w"][0], 1e-6, out_dtype=F32)
    torch.cuda.synchronize()
    for n in (0, N // 3, N - 2, N - 1):
        y_ref = oracle.rmsnorm_gate(x["o"][n].cpu(), x["g"][n].cpu(), x["w"][0].cpu(), eps=1e-6)
        e = _err(y[n].cpu(), y_ref)
        print(f"  rows of token {n}: err(y)={e:.2e}")
        assert e <= 1e-3, (n, e)
