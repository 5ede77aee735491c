"""GPU parity of the solved-probe decode (parallax_decode_lla) against the
fp64 oracle, through the C ABI: the probe rho* = (S_KK + lam I)^{-1} (kbar - q)
that conjugate gradients reach (each step one decode sweep with the keys as
values) and the Parallax output with it.

Tolerance: the sweeps are the decode kernels, accurate to about 1e-6
(fp32 cache) or 2^-16 (bf16 cache, two-term bf16 operands) relative; CG
reaches the fixed point of that arithmetic, so the probe's relative error is
about the condition number of S_KK + lam I (below 10 for these inputs at
lam = 0.5) times that: bounds of 1e-4 (fp32) and 1e-3 (bf16) keep a margin
of about 10.
"""
import numpy as np
import pytest
import torch

import oracle
import parallax_local_linear_decode_amd as plx
from parallax_local_linear_decode_amd.workloads import decode_inputs, host_array, paged_inputs

from helpers import assert_parity

pytestmark = pytest.mark.gpu

TAU = {torch.float32: 1e-4, torch.bfloat16: 1e-3}


def to(inp, dev):
    for name in ("q", "rho", "k", "v", "seq_lens", "block_table"):
        t = getattr(inp, name)
        if t is not None:
            setattr(inp, name, t.to(dev))
    return inp


def oracle_lla(inp, lam, window=0):
    sl = None if inp.seq_lens is None else host_array(inp.seq_lens).astype(np.int32)
    bt = None if inp.block_table is None else host_array(inp.block_table)
    return oracle.lla_decode(host_array(inp.q), host_array(inp.k), host_array(inp.v), inp.scale,
                             lam, seq_lens=sl, block_table=bt, window=window)


def run(inp, lam, iterations, **kw):
    out, rho, resid = plx.parallax_decode_lla(inp.q, inp.k, inp.v, lam=lam,
                                              iterations=iterations, scale=inp.scale,
                                              seq_lens=inp.seq_lens,
                                              block_table=inp.block_table, **kw)
    torch.cuda.synchronize()
    return out, rho, resid


@pytest.mark.parametrize("kv_dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("G", [1, 2, 4, 8])
def test_ragged_rows(gpu, kv_dtype, d, G):
    lens = [0, 1, 2, 3, 17, 33, 64, 129, 200, 300]
    inp = decode_inputs(len(lens), 2 * G, 2, d, 304, kv_dtype=kv_dtype, seed=G * 3 + d)
    inp.seq_lens = torch.tensor(lens, dtype=torch.int32)
    ref_out, ref_rho = oracle_lla(inp, 0.5)
    out, rho, resid = run(to(inp, gpu), 0.5, 64)
    tau = TAU[kv_dtype]
    assert_parity(rho, ref_rho, tau, tau, what="rho*")
    assert_parity(out, ref_out, tau, tau, what="out")
    assert torch.all(out[0] == 0) and torch.all(rho[0] == 0) and torch.all(resid[0] == 0)
    assert resid.max().item() < tau


@pytest.mark.parametrize("lam", [0.1, 2.0])
def test_lambda_and_window(gpu, lam):
    inp = decode_inputs(4, 8, 4, 128, 600, seed=int(lam * 10))
    inp.seq_lens = torch.tensor([600, 450, 37, 1], dtype=torch.int32)
    for W in (0, 16, 100):
        ref_out, ref_rho = oracle_lla(inp, lam, window=W)
        out, rho, _ = run(to(inp, gpu), lam, 96, window=W)
        assert_parity(rho, ref_rho, TAU[torch.bfloat16], TAU[torch.bfloat16],
                      what=f"lam={lam} W={W} rho*")
        assert_parity(out, ref_out, TAU[torch.bfloat16], TAU[torch.bfloat16],
                      what=f"lam={lam} W={W} out")


def test_paged(gpu):
    inp = paged_inputs(12, 16, 8, 128, ctx_lo=1, ctx_hi=700, seed=50, rho_zero_rows=0)
    ref_out, ref_rho = oracle_lla(inp, 0.5)
    out, rho, _ = run(to(inp, gpu), 0.5, 48)
    assert_parity(rho, ref_rho, TAU[torch.bfloat16], TAU[torch.bfloat16], what="paged rho*")
    assert_parity(out, ref_out, TAU[torch.bfloat16], TAU[torch.bfloat16], what="paged out")


def test_large_lambda_is_softmax(gpu):
    """A regulariser far above S_KK makes rho* ~ 0: the output is the plain
    softmax output (parallax_decode with rho = 0)."""
    inp = to(decode_inputs(2, 8, 4, 128, 300, seed=51), gpu)
    out, rho, _ = run(inp, 1e6, 8)
    soft = plx.parallax_decode(inp.q, torch.zeros_like(inp.q), inp.k, inp.v, scale=inp.scale)
    assert rho.abs().max().item() < 1e-4
    assert (out - soft).abs().max().item() < 1e-4


def test_deterministic_and_workspace_contents_do_not_matter(gpu):
    inp = to(decode_inputs(3, 16, 8, 128, 1000, seed=52), gpu)
    first = [t.clone() for t in run(inp, 0.5, 20)]
    for fill in (0, 255):
        ws = torch.full((1 << 22,), fill, dtype=torch.uint8, device=gpu)
        again = run(inp, 0.5, 20, workspace=ws)
        for a, b in zip(first, again):
            assert torch.equal(a, b)


def test_more_iterations_lower_the_residual(gpu):
    inp = to(decode_inputs(2, 8, 4, 128, 2000, seed=53), gpu)
    res = [run(inp, 0.2, n)[2].max().item() for n in (1, 4, 16)]
    assert res[0] > res[1] > res[2]


@pytest.mark.slow
def test_full_size(gpu):
    """Batch 8 x 4096 tokens, 16 query / 8 KV heads, d 128, bf16 cache; the
    oracle on sequences 0 and 5 (every head)."""
    inp = decode_inputs(8, 16, 8, 128, 4096, seed=54)
    sub = decode_inputs(8, 16, 8, 128, 4096, seed=54)
    out, rho, resid = run(to(inp, gpu), 0.5, 32)
    idx = torch.tensor([0, 5])
    for name in ("q", "k", "v"):
        setattr(sub, name, getattr(sub, name)[idx])
    ref_out, ref_rho = oracle_lla(sub, 0.5)
    assert_parity(rho[idx.to(gpu)], ref_rho, TAU[torch.bfloat16], TAU[torch.bfloat16],
                  what="full rho*")
    assert_parity(out[idx.to(gpu)], ref_out, TAU[torch.bfloat16], TAU[torch.bfloat16],
                  what="full out")
    assert resid.max().item() < 1e-3


def test_graph_replay(gpu):
    """The whole solved-probe call (iterations + 2 decode sweeps and the
    vector kernels, no host synchronisation, no memsets) captured once in a
    HIP graph replays to the eager result, with eager calls in between."""
    inp = to(decode_inputs(3, 16, 8, 128, 1500, seed=55), gpu)
    ws = torch.zeros(1 << 22, dtype=torch.uint8, device=gpu)
    bufs = [torch.empty((3, 16, 128), dtype=torch.float32, device=gpu) for _ in range(2)]
    resid = torch.empty((3, 16), dtype=torch.float32, device=gpu)
    want = [t.clone() for t in run(inp, 0.5, 12, workspace=ws)]
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        run(inp, 0.5, 12, workspace=ws, out=bufs[0], rho_out=bufs[1], resid=resid)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            plx.parallax_decode_lla(inp.q, inp.k, inp.v, lam=0.5, iterations=12,
                                    scale=inp.scale, out=bufs[0], rho_out=bufs[1], resid=resid,
                                    workspace=ws)
    other = to(decode_inputs(2, 8, 4, 128, 700, seed=56), gpu)
    for r in range(4):
        for t in (*bufs, resid):
            t.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        for a, b in zip(want, (bufs[0], bufs[1], resid)):
            assert torch.equal(a, b), f"replay {r}"
        run(other, 0.3, 5, workspace=ws)  # an eager call of another shape in between
