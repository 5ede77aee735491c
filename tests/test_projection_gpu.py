"""GPU parity of parallax_qr_projection (q = W_Q x and rho = W_R x in one
launch) against the oracle's fp64 products, through the C ABI, and its use as
the input of decode and prefill through strided views.

Tolerance: bf16 inputs are exact matrix-core operands and the sums run in
fp32 over D terms, so fp32 outputs are within a few fp32 ulps of the sum of
|terms| (bound 1e-5 (1 + |ref|) at D <= 4096 for these inputs); bf16 outputs
add one rounding, 2^-9 relative (bound 2^-8 (1 + |ref|)).
"""
import numpy as np
import pytest
import torch

import oracle
import parallax_local_linear_decode_amd as plx
from parallax_local_linear_decode_amd.workloads import decode_inputs, host_array

from helpers import RMS_DECODE_BF16, TAU_BF16, assert_parity

pytestmark = pytest.mark.gpu


def weights(T, D, N, seed, dev):
    g = torch.Generator(device="cpu").manual_seed(seed)
    x = torch.randn((T, D), generator=g).to(torch.bfloat16)
    w_q = (torch.randn((N, D), generator=g) / D ** 0.5).to(torch.bfloat16)
    w_r = (torch.randn((N, D), generator=g) / D ** 0.5).to(torch.bfloat16)
    return x.to(dev), w_q.to(dev), w_r.to(dev)


@pytest.mark.parametrize("T", [1, 8, 16, 17, 64, 100, 300])
@pytest.mark.parametrize("D,Hq,d", [(256, 2, 64), (2048, 16, 128), (1280, 4, 64)])
@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_every_element(gpu, T, D, Hq, d, out_dtype):
    x, w_q, w_r = weights(T, D, Hq * d, T * 7 + D, gpu)
    q, rho = plx.parallax_qr_projection(x, w_q, w_r, num_q_heads=Hq, out_dtype=out_dtype)
    torch.cuda.synchronize()
    rq, rr = oracle.qr_projection(host_array(x), host_array(w_q), host_array(w_r))
    tau = 1e-5 if out_dtype == torch.float32 else 2.0 ** -8
    assert_parity(q.reshape(T, -1), rq, tau, what="q")
    assert_parity(rho.reshape(T, -1), rr, tau, what="rho")


@pytest.mark.parametrize("T,D,Hq,d", [(4096, 2048, 16, 128), (4100, 1024, 16, 128),
                                      (4100, 8192, 16, 128), (8200, 512, 8, 128),
                                      (32900, 256, 2, 128), (22000, 256, 3, 128),
                                      (4100, 256, 1, 64)])
@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_prefill_token_counts(gpu, T, D, Hq, d, out_dtype):
    """Token counts of prefill, the LDS-tiled GEMMs with ragged last token
    tiles: the four-wave 256 x 256 kernel (N a multiple of 256; model dims 256
    to 8192, i.e. 4 to 128 chunks through its two LDS stages; the 32900-token
    grid of 258 tiles is not a multiple of eight, so its tiles keep launch
    order), the eight-wave 256 x 256 kernel (N = 384) and 128 x 128 tiles
    (Hq = 1, d = 64).  Sampled rows against the oracle: the first and last
    tiles and rows across tile edges."""
    x, w_q, w_r = weights(T, D, Hq * d, T + D + Hq, gpu)
    q, rho = plx.parallax_qr_projection(x, w_q, w_r, num_q_heads=Hq, out_dtype=out_dtype)
    torch.cuda.synchronize()
    rows = sorted(set(range(64)) | set(range(250, 262)) | set(range(2040, 2060)) |
                  set(range(T - 70, T)))
    idx = torch.tensor(rows)
    rq, rr = oracle.qr_projection(host_array(x[idx.to(gpu)]), host_array(w_q), host_array(w_r))
    tau = 1e-5 if out_dtype == torch.float32 else 2.0 ** -8
    assert_parity(q[idx.to(gpu)].reshape(len(rows), -1), rq, tau, what="q")
    assert_parity(rho[idx.to(gpu)].reshape(len(rows), -1), rr, tau, what="rho")


def test_prefill_token_counts_into_strided_views(gpu):
    """The 256 x 256 tiled GEMM writing bf16 q and rho into the two halves of
    one [T, 2, Hq, d] buffer (row stride 2 Hq d): equal to contiguous outputs."""
    T, D, Hq, d = 4200, 1024, 16, 128
    x, w_q, w_r = weights(T, D, Hq * d, 76, gpu)
    buf = torch.full((T, 2, Hq, d), float("nan"), dtype=torch.bfloat16, device=gpu)
    q, rho = plx.parallax_qr_projection(x, w_q, w_r, num_q_heads=Hq, out_dtype=torch.bfloat16,
                                        q=buf[:, 0], rho=buf[:, 1])
    qc, rc = plx.parallax_qr_projection(x, w_q, w_r, num_q_heads=Hq, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert torch.equal(q, qc) and torch.equal(rho, rc)
    assert not torch.isnan(buf.float()).any()


@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_prefill_token_counts_strided_x(gpu, out_dtype):
    """x as a column slice of a wider buffer (row stride 1536, offset 256):
    the four-wave kernel's buffer bounds follow the stride; equal to the
    contiguous copy's result bit for bit."""
    T, D, Hq, d = 4100, 1024, 16, 128
    x, w_q, w_r = weights(T, D, Hq * d, 77, gpu)
    wide = torch.full((T, 1536), float("nan"), dtype=torch.bfloat16, device=gpu)
    wide[:, 256:256 + D] = x
    xs = wide[:, 256:256 + D]
    q, rho = plx.parallax_qr_projection(xs, w_q, w_r, num_q_heads=Hq, out_dtype=out_dtype)
    qc, rc = plx.parallax_qr_projection(x, w_q, w_r, num_q_heads=Hq, out_dtype=out_dtype)
    torch.cuda.synchronize()
    assert torch.equal(q, qc) and torch.equal(rho, rc)


def test_zero_probe_weights_give_zero_rho(gpu):
    x, w_q, w_r = weights(8, 2048, 2048, 70, gpu)
    _, rho = plx.parallax_qr_projection(x, w_q, torch.zeros_like(w_r), num_q_heads=16)
    torch.cuda.synchronize()
    assert torch.all(rho == 0)


def test_into_strided_views_feeds_decode(gpu):
    """q and rho written into one [B, 2, Hq, d] buffer (the layout of a
    stacked projection), then read by parallax_decode through their strides."""
    B, Hq, Hkv, d, D = 8, 16, 8, 128, 2048
    x, w_q, w_r = weights(B, D, Hq * d, 71, gpu)
    buf = torch.full((B, 2, Hq, d), float("nan"), dtype=torch.float32, device=gpu)
    q, rho = plx.parallax_qr_projection(x, w_q, w_r, num_q_heads=Hq, q=buf[:, 0], rho=buf[:, 1])
    inp = decode_inputs(B, Hq, Hkv, d, 700, seed=72)
    k, v = inp.k.to(gpu), inp.v.to(gpu)
    out = plx.parallax_decode(q, rho, k, v, scale=inp.scale)
    torch.cuda.synchronize()
    rq, rr = oracle.qr_projection(host_array(x), host_array(w_q), host_array(w_r))
    ref = oracle.decode(rq.reshape(B, Hq, d), rr.reshape(B, Hq, d), host_array(inp.k),
                        host_array(inp.v), inp.scale)
    assert_parity(out, ref, TAU_BF16, RMS_DECODE_BF16, what="decode from projection")


def test_deterministic(gpu):
    x, w_q, w_r = weights(300, 2048, 2048, 73, gpu)
    a = [t.clone() for t in plx.parallax_qr_projection(x, w_q, w_r, num_q_heads=16)]
    for _ in range(5):
        b = plx.parallax_qr_projection(x, w_q, w_r, num_q_heads=16)
        torch.cuda.synchronize()
        assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def test_projection_feeds_prefill(gpu):
    """x -> (q, rho) in bf16 straight into one [T, 2, Hq, d] buffer -> causal
    prefill through strided views, against the oracle chain (projection, then
    prefill on the same bf16-rounded q and rho)."""
    B, S, Hq, Hkv, d, D = 1, 200, 4, 2, 128, 512
    x, w_q, w_r = weights(B * S, D, Hq * d, 74, gpu)
    # rho ~ N(0, 0.1^2) as in the prefill workload (the prefill tolerance
    # assumes a probe of that size)
    w_r = (w_r.float() * 0.1).to(torch.bfloat16)
    buf = torch.empty((B * S, 2, Hq, d), dtype=torch.bfloat16, device=gpu)
    q, rho = plx.parallax_qr_projection(x, w_q, w_r, num_q_heads=Hq, out_dtype=torch.bfloat16,
                                        q=buf[:, 0], rho=buf[:, 1])
    g = torch.Generator(device="cpu").manual_seed(75)
    k = torch.randn((B, S, Hkv, d), generator=g).to(torch.bfloat16).to(gpu)
    v = torch.randn((B, S, Hkv, d), generator=g).to(torch.bfloat16).to(gpu)
    out = plx.parallax_prefill(q.view(B, S, Hq, d), rho.view(B, S, Hq, d), k, v, scale=d ** -0.5)
    torch.cuda.synchronize()
    rq, rr = oracle.qr_projection(host_array(x), host_array(w_q), host_array(w_r))
    # the oracle prefill sees the projection rounded to bf16 as the kernel wrote it
    qb = host_array(q.contiguous()).reshape(B, S, Hq, d)
    rb = host_array(rho.contiguous()).reshape(B, S, Hq, d)
    assert_parity(q.reshape(B * S, -1), rq, 2.0 ** -8, what="q")
    assert_parity(rho.reshape(B * S, -1), rr, 2.0 ** -8, what="rho")
    ref = oracle.prefill(qb, rb, host_array(k), host_array(v), d ** -0.5)
    assert_parity(out, ref, TAU_BF16, 1e-2, what="prefill from projection")
