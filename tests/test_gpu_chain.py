"""The Mamba-2 mixer chain on the GPU: causal conv1d -> SSD forward -> gated
RMSNorm (page "ops-transformer MambaV2 算子套件" §2: the operator chain, with
§4.1 before and §4.6 after the SSD), end to end against the chain of fp64
oracles, and captured as one HIP graph whose replays equal the eager run bit
for bit.  Also a captured backward.

The chain moves no data between the kernels: the projection row of a token
holds xBC and dt side by side ([B, L, H*P + 2*G*N + H]); the token-major conv
reads its xBC columns and writes xbc [B, L, H*P + 2*G*N]; the SSD reads x, B
and C as column views of xbc and dt as a column view of the projection row.

Chain bar: the SSD's fp16-operand bound, max|gpu - oracle| <= 2e-3 *
max|oracle| on the normalised output (the conv and the norm are fp32 and
add errors below 1e-5 of their outputs; the norm does not amplify relative
errors beyond a factor of order one).
"""
import sys

import numpy as np
import pytest
import torch

from oracle import causal_conv1d as oracle_conv
from oracle import rmsnorm_gated as oracle_norm
from oracle import ssd_recurrence
from workloads import NORM_EPS, conv_inputs, random_inputs

pytestmark = pytest.mark.gpu

Bsz, L, H, P, N, G, Q = 2, 640, 4, 64, 64, 2, 128
DC = H * P + 2 * G * N


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _inputs():
    conv = conv_inputs(Bsz, DC, L, 4, seed=901, device="cpu", has_state=True)
    d = random_inputs(Bsz, L, H, P, N, G, seed=902, has_D=True, has_z=True, has_h0=True)
    g = torch.Generator().manual_seed(903)
    normw = 1.0 + 0.1 * torch.randn(H * P, generator=g)
    return conv, d, normw


class Chain:
    """Buffers fixed up front, so that one call allocates nothing."""

    def __init__(self, ssd, conv, d, normw):
        cu = lambda t: None if t is None else t.cuda()
        self.ssd = ssd
        self.conv = {k: cu(v) for k, v in conv.items()}
        self.d = {k: cu(v) for k, v in d.items()}
        self.normw = normw.cuda()
        # the projection rows: xBC (the conv's input) then dt
        self.proj = torch.empty(Bsz, L, DC + H, device="cuda")
        self.proj[..., :DC] = self.conv["x"].transpose(1, 2)
        self.proj[..., DC:] = self.d["dt"]
        self.xbc = torch.empty(Bsz, L, DC, device="cuda")
        self.cfin = torch.empty(Bsz, DC, 3, device="cuda")
        hp, gn = H * P, G * N
        x = self.xbc[..., :hp].view(Bsz, L, H, P)
        Bv = self.xbc[..., hp:hp + gn].view(Bsz, L, G, N)
        Cv = self.xbc[..., hp + gn:].view(Bsz, L, G, N)
        dt = self.proj[..., DC:]
        self.normed = torch.empty(Bsz * L, H * P, device="cuda")
        self.call, self.out, self.fin, self.ws = ssd.prepare(
            x, dt, self.d["A"], Bv, Cv, Q, D=self.d["D"],
            initial_states=self.d["initial_states"], dt_softplus=True, return_final_state=True)

    def run(self, stream):
        c = self.conv
        self.ssd.causal_conv1d_tokmajor(self.proj[..., :DC], c["w"], c["bias"], c["conv_state"],
                                        out=self.xbc, return_final_state=True,
                                        final_state=self.cfin)
        self.call.launch(stream)
        self.ssd.rmsnorm_gated(self.out.view(Bsz * L, H * P), self.d["z"].view(Bsz * L, H * P),
                               self.normw, G, NORM_EPS, out=self.normed)


def test_chain_matches_the_oracle_chain(gpu_lib):
    conv, d, normw = _inputs()
    ch = Chain(gpu_lib, conv, d, normw)
    ch.run(torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    xbc, _ = oracle_conv(conv["x"].numpy(), conv["w"].numpy(), conv["bias"].numpy(),
                         conv["conv_state"].numpy())
    t = np.transpose(xbc, (0, 2, 1))
    x = t[..., :H * P].reshape(Bsz, L, H, P)
    Bm = t[..., H * P:H * P + G * N].reshape(Bsz, L, G, N)
    Cm = t[..., H * P + G * N:].reshape(Bsz, L, G, N)
    y, _ = ssd_recurrence(x, d["dt"], d["A"], Bm, Cm, D=d["D"],
                          initial_states=d["initial_states"], dt_softplus=True)
    ref = oracle_norm(y.reshape(Bsz * L, H * P), d["z"].numpy().reshape(Bsz * L, H * P),
                      normw.numpy(), G, NORM_EPS)
    got = ch.normed.cpu().double().numpy()
    e = float(np.abs(got - ref).max() / np.abs(ref).max())
    _say(f"    chain: max_err/max_ref={e:.3e}")
    assert e <= 2e-3


def test_chain_in_one_graph_replays_bit_identically(gpu_lib):
    conv, d, normw = _inputs()
    ch = Chain(gpu_lib, conv, d, normw)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        ch.run(s.cuda_stream)
    torch.cuda.synchronize()
    ref = ch.normed.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        ch.run(s.cuda_stream)
    for k in range(3):
        ch.normed.fill_(float("nan"))
        ch.xbc.fill_(float("nan"))
        junk = torch.randn(1 << 20, device="cuda").sum()   # unrelated eager work
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(ch.normed, ref), f"replay {k} differs"
        del junk


def test_backward_in_a_graph_replays_bit_identically(gpu_lib):
    d = {k: (None if v is None else v.cuda())
         for k, v in random_inputs(2, 300, 4, 64, 64, 2, seed=904, has_D=True, has_z=True,
                                   has_h0=True, dt_bias=True).items()}
    gdo = torch.Generator(device="cuda").manual_seed(905)
    dout = torch.randn(2, 300, 4, 64, device="cuda", generator=gdo)
    call = gpu_lib.prepare_bwd(d["x"], d["dt"], d["A"], d["B"], d["C"], dout, 64, D=d["D"],
                               z=d["z"], dt_bias=d["dt_bias"],
                               initial_states=d["initial_states"], dt_softplus=True)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        call.launch(s.cuda_stream)
    torch.cuda.synchronize()
    ref = {k: v.clone() for k, v in call.grads.items() if v is not None}
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        call.launch(s.cuda_stream)
    for k in range(3):
        for v in call.grads.values():
            if v is not None:
                v.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for name, v in ref.items():
            assert torch.equal(call.grads[name], v), f"replay {k}: {name} differs"
