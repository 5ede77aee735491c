"""GPU parity of the causal prefill backward pass (parallax_prefill_backward)
and of the statistics the forward pass keeps for it, against the fp64 oracle,
through the C ABI.

The GPU backward consumes the GPU forward's own outputs (out, o_sa, lse, r);
the oracle recomputes everything from the inputs, so these tests check the
whole training step.  Small cases compare every element (ragged lengths
around the 32-row tiles and 128-row blocks, GQA groups 1/2/4/8/16, local windows,
head dims 128 and 64);
the full-size workload (batch 4 x 8192 tokens, 16 query / 8 KV heads, d 128)
compares sampled rows of dq and drho, the last 64 keys' dk and dv (exact for
them: no earlier row sees those keys), and two properties that hold at any
size: per (batch, KV head) the value gradients sum to the summed dout of its
rows, and the key gradients sum to zero.
"""
import numpy as np
import pytest
import torch

import oracle
import parallax_local_linear_decode_amd as plx
from parallax_local_linear_decode_amd.workloads import host_array, prefill_dout, prefill_inputs

from helpers import RMS_BWD, RMS_PREFILL, TAU_BF16, TAU_BWD, assert_parity

pytestmark = pytest.mark.gpu

# log-sum-exp: the forward's denominator sums bf16-rounded numerators, each
# within 2^-9 relative, so log Z is within about 2e-3 of the exact value.
LSE_ABS = 4e-3


def forward_backward(q, rho, k, v, dout, scale, window=0):
    out, lse, rmean, o_sa = plx.parallax_prefill(q, rho, k, v, scale=scale, window=window,
                                                 return_stats=True)
    grads = plx.parallax_prefill_backward(q, rho, k, v, dout, out, o_sa, lse, rmean,
                                          scale=scale, window=window)
    torch.cuda.synchronize()
    return (out, lse, rmean, o_sa), grads


def case(B, S, Hq, Hkv, seed, device, d=128):
    q, rho, k, v, scale = prefill_inputs(B, S, Hq, Hkv, d, seed=seed, device=device)
    dout = prefill_dout(B, S, Hq, d, seed=seed + 7919, device=device)
    return q, rho, k, v, dout, scale


def check_stats(stats, q, rho, k, v, scale, window=0, rows=None, what=""):
    out, lse, rmean, o_sa = stats
    h = [host_array(t) for t in (q, rho, k, v)]
    ref_lse, ref_r, ref_a = oracle.prefill_stats(*h, scale, rows=rows, window=window)
    sel = slice(None) if rows is None else torch.as_tensor(rows, dtype=torch.long)
    got_lse = lse[:, :, sel].permute(0, 2, 1).double().cpu().numpy()
    got_r = rmean[:, :, sel].permute(0, 2, 1)
    assert np.all(np.isfinite(got_lse))
    err = float(np.max(np.abs(got_lse - ref_lse)))
    assert err <= LSE_ABS, f"{what}: lse err {err:.2e}"
    assert_parity(got_r, ref_r, TAU_BF16, RMS_PREFILL, what=f"{what} r")
    assert_parity(o_sa[:, sel], ref_a, TAU_BF16, RMS_PREFILL, what=f"{what} o_sa")


@pytest.mark.parametrize("d", [128, 64])
@pytest.mark.parametrize("S", [1, 17, 31, 32, 33, 64, 100, 129, 257])
@pytest.mark.parametrize("Hq,Hkv", [(2, 1), (4, 2), (2, 2), (8, 2), (8, 1), (16, 2), (16, 1)])
def test_small_every_gradient(gpu, S, Hq, Hkv, d):
    q, rho, k, v, dout, scale = case(2, S, Hq, Hkv, S * 10 + Hq + d, gpu, d)
    stats, grads = forward_backward(q, rho, k, v, dout, scale)
    what = f"S={S} {Hq}/{Hkv} d={d}"
    check_stats(stats, q, rho, k, v, scale, what=what)
    ref = oracle.prefill_backward(*(host_array(t) for t in (q, rho, k, v, dout)), scale)
    for name, g, r in zip(("dq", "drho", "dk", "dv"), grads, ref):
        assert_parity(g, r, TAU_BWD, RMS_BWD, what=f"{what} {name}")


@pytest.mark.parametrize("W", [1, 5, 31, 32, 33, 100])
@pytest.mark.parametrize("S,Hq,Hkv,d", [(100, 4, 2, 128), (300, 2, 1, 128), (257, 8, 2, 128),
                                        (300, 4, 2, 64), (200, 16, 2, 128), (150, 16, 1, 64)])
def test_window_every_gradient(gpu, S, Hq, Hkv, d, W):
    q, rho, k, v, dout, scale = case(1, S, Hq, Hkv, S + W, gpu, d)
    stats, grads = forward_backward(q, rho, k, v, dout, scale, window=W)
    what = f"S={S} W={W} d={d}"
    check_stats(stats, q, rho, k, v, scale, window=W, what=what)
    ref = oracle.prefill_backward(*(host_array(t) for t in (q, rho, k, v, dout)), scale,
                                  window=W)
    for name, g, r in zip(("dq", "drho", "dk", "dv"), grads, ref):
        assert_parity(g, r, TAU_BWD, RMS_BWD, what=f"{what} {name}")


def test_head_dim_64_larger(gpu):
    """d 64 over several 128-key blocks: batch 2 x 1500 tokens, 8 query / 2
    KV heads; sampled rows of dq and drho, the last 64 keys' dk and dv."""
    B, S, Hq, Hkv = 2, 1500, 8, 2
    q, rho, k, v, dout, scale = case(B, S, Hq, Hkv, 64, gpu, 64)
    stats, (dq, drho, dk, dv) = forward_backward(q, rho, k, v, dout, scale)
    rows = np.array([0, 1, 31, 32, 127, 128, 700, 1023, 1024] + list(range(S - 64, S)),
                    dtype=np.int32)
    h = [host_array(t) for t in (q, rho, k, v, dout)]
    check_stats(stats, q, rho, k, v, scale, rows=rows, what="d=64")
    r_dq, r_drho, r_dk, r_dv = oracle.prefill_backward(*h, scale, rows=rows)
    sel = torch.as_tensor(rows, dtype=torch.long)
    assert_parity(dq[:, sel], r_dq, TAU_BWD, RMS_BWD, what="d=64 dq")
    assert_parity(drho[:, sel], r_drho, TAU_BWD, RMS_BWD, what="d=64 drho")
    assert_parity(dk[:, S - 64:], r_dk[:, S - 64:], TAU_BWD, RMS_BWD, what="d=64 dk tail")
    assert_parity(dv[:, S - 64:], r_dv[:, S - 64:], TAU_BWD, RMS_BWD, what="d=64 dv tail")
    g_sum = dout.double().reshape(B, S, Hkv, Hq // Hkv, 64).sum(dim=(1, 3)).cpu().numpy()
    assert_parity(dv.double().sum(dim=1), g_sum, TAU_BWD, RMS_BWD, what="d=64 sum dv")


def test_window_at_least_the_sequence_is_full(gpu):
    q, rho, k, v, dout, scale = case(1, 200, 4, 2, 11, gpu)
    _, full = forward_backward(q, rho, k, v, dout, scale)
    full = [t.clone() for t in full]
    for W in (200, 5000):
        _, win = forward_backward(q, rho, k, v, dout, scale, window=W)
        for a, b in zip(full, win):
            assert torch.equal(a, b)


def test_rho_zero_matches_softmax_attention_gradients(gpu):
    """rho = 0: dq, dk, dv are those of plain causal softmax attention
    (torch autograd in fp64 on the CPU)."""
    q, rho, k, v, dout, scale = case(1, 150, 4, 2, 12, gpu)
    rho = torch.zeros_like(rho)
    _, grads = forward_backward(q, rho, k, v, dout, scale)
    tq, tk, tv = (t.double().cpu().requires_grad_() for t in (q, k, v))
    o = torch.nn.functional.scaled_dot_product_attention(
        tq.transpose(1, 2), tk.repeat_interleave(2, dim=2).transpose(1, 2),
        tv.repeat_interleave(2, dim=2).transpose(1, 2), is_causal=True, scale=scale)
    (o.transpose(1, 2) * dout.double().cpu()).sum().backward()
    for name, g, r in (("dq", grads[0], tq.grad), ("dk", grads[2], tk.grad),
                       ("dv", grads[3], tv.grad)):
        assert_parity(g, r.numpy(), TAU_BWD, RMS_BWD, what=f"rho=0 {name}")


def test_strided_views_and_preallocated_outputs(gpu):
    """Inputs as views into wider buffers and caller-owned outputs (given
    garbage first) give the same bits as contiguous tensors."""
    q, rho, k, v, dout, scale = case(1, 96, 4, 2, 13, gpu)
    _, ref = forward_backward(q, rho, k, v, dout, scale)
    wide = torch.zeros((1, 96, 4, 256), dtype=torch.bfloat16, device=gpu)
    wide[..., 64:192] = q
    qv = wide[..., 64:192]
    stats = plx.parallax_prefill(qv, rho, k, v, scale=scale, return_stats=True)
    outs = [torch.full_like(t, float("nan")) for t in ref]
    ws = torch.full((1 << 16,), 255, dtype=torch.uint8, device=gpu)
    got = plx.parallax_prefill_backward(qv, rho, k, v, dout, *stats[:1], stats[3], stats[1],
                                        stats[2], scale=scale, dq=outs[0], drho=outs[1],
                                        dk=outs[2], dv=outs[3], workspace=ws)
    torch.cuda.synchronize()
    for a, b in zip(ref, got):
        assert torch.equal(a, b)


def test_deterministic_small(gpu):
    q, rho, k, v, dout, scale = case(2, 300, 8, 2, 14, gpu)
    _, first = forward_backward(q, rho, k, v, dout, scale)
    first = [t.clone() for t in first]
    for _ in range(10):
        _, again = forward_backward(q, rho, k, v, dout, scale)
        for a, b in zip(first, again):
            assert torch.equal(a, b)


@pytest.mark.slow
def test_full_size(gpu):
    B, S, Hq, Hkv = 4, 8192, 16, 8
    q, rho, k, v, dout, scale = case(B, S, Hq, Hkv, 15, gpu)
    stats, grads = forward_backward(q, rho, k, v, dout, scale)
    dq, drho, dk, dv = grads
    for t in grads:
        assert torch.isfinite(t).all()
    rng = np.random.default_rng(15)
    early = [0, 1, 31, 32, 127, 128, 1000, 4095, 4096] + sorted(rng.integers(0, S - 64, 12))
    tail = list(range(S - 64, S))
    rows = np.array(sorted(set(early)) + tail, dtype=np.int32)
    # the oracle on sequences 0 and 3 (every head), to bound its CPU time
    bs = [0, 3]
    sub = [t[bs] for t in (q, rho, k, v, dout)]
    check_stats([t[bs] for t in stats], *sub[:4], scale, rows=rows, what="full size")
    r_dq, r_drho, r_dk, r_dv = oracle.prefill_backward(*(host_array(t) for t in sub), scale,
                                                       rows=rows)
    sel = torch.as_tensor(rows, dtype=torch.long)
    assert_parity(dq[bs][:, sel], r_dq, TAU_BWD, RMS_BWD, what="full dq")
    assert_parity(drho[bs][:, sel], r_drho, TAU_BWD, RMS_BWD, what="full drho")
    assert_parity(dk[bs, S - 64:], r_dk[:, S - 64:], TAU_BWD, RMS_BWD, what="full dk tail")
    assert_parity(dv[bs, S - 64:], r_dv[:, S - 64:], TAU_BWD, RMS_BWD, what="full dv tail")
    # invariants over every key
    g_sum = dout.double().reshape(B, S, Hkv, Hq // Hkv, 128).sum(dim=(1, 3)).cpu().numpy()
    assert_parity(dv.double().sum(dim=1), g_sum, TAU_BWD, RMS_BWD, what="sum dv")
    dk_sum = dk.double().sum(dim=1).abs().max().item()
    dk_scale = dk.double().abs().sum(dim=1).max().item()
    assert dk_sum <= 1e-3 * dk_scale, (dk_sum, dk_scale)


@pytest.mark.slow
def test_long_sequence(gpu):
    """One sequence of 32768 tokens (16/8 heads, d 128): sampled rows of dq
    and drho, the last 32 keys' dk and dv (exact from the last 32 rows)."""
    B, S, Hq, Hkv = 1, 32768, 16, 8
    q, rho, k, v, dout, scale = case(B, S, Hq, Hkv, 22, gpu)
    _, (dq, drho, dk, dv) = forward_backward(q, rho, k, v, dout, scale)
    rng = np.random.default_rng(22)
    rows = np.array(sorted(set([0, 127, 128, 16384] + list(rng.integers(0, S - 32, 4)) +
                               list(range(S - 32, S)))), dtype=np.int32)
    h = [host_array(t) for t in (q, rho, k, v, dout)]
    r_dq, r_drho, r_dk, r_dv = oracle.prefill_backward(*h, scale, rows=rows)
    sel = torch.as_tensor(rows, dtype=torch.long)
    assert_parity(dq[:, sel], r_dq, TAU_BWD, RMS_BWD, what="32768 dq")
    assert_parity(drho[:, sel], r_drho, TAU_BWD, RMS_BWD, what="32768 drho")
    assert_parity(dk[:, S - 32:], r_dk[:, S - 32:], TAU_BWD, RMS_BWD, what="32768 dk tail")
    assert_parity(dv[:, S - 32:], r_dv[:, S - 32:], TAU_BWD, RMS_BWD, what="32768 dv tail")


@pytest.mark.slow
def test_full_size_deterministic(gpu):
    q, rho, k, v, dout, scale = case(4, 8192, 16, 8, 16, gpu)
    stats, first = forward_backward(q, rho, k, v, dout, scale)
    first = [t.clone() for t in first]
    for _ in range(5):
        grads = plx.parallax_prefill_backward(q, rho, k, v, dout, stats[0], stats[3], stats[1],
                                              stats[2], scale=scale)
        torch.cuda.synchronize()
        for a, b in zip(first, grads):
            assert torch.equal(a, b)


@pytest.mark.slow
def test_full_size_window(gpu):
    B, S, Hq, Hkv, W = 4, 8192, 16, 8, 1024
    q, rho, k, v, dout, scale = case(B, S, Hq, Hkv, 17, gpu)
    _, (dq, drho, dk, dv) = forward_backward(q, rho, k, v, dout, scale, window=W)
    # rows 3000..4063 are every row that sees keys 3000..3040 (window 1024);
    # the oracle on sequence 1, every head
    rows = np.arange(3000, 3000 + 40 + W, dtype=np.int32)
    sub = [t[1:2] for t in (q, rho, k, v, dout)]
    r_dq, r_drho, r_dk, r_dv = oracle.prefill_backward(*(host_array(t) for t in sub), scale,
                                                       rows=rows, window=W)
    sel = torch.as_tensor(rows, dtype=torch.long)
    assert_parity(dq[1:2, sel], r_dq, TAU_BWD, RMS_BWD, what="window dq")
    assert_parity(drho[1:2, sel], r_drho, TAU_BWD, RMS_BWD, what="window drho")
    assert_parity(dk[1:2, 3000:3040], r_dk[:, 3000:3040], TAU_BWD, RMS_BWD,
                  what="window dk")
    assert_parity(dv[1:2, 3000:3040], r_dv[:, 3000:3040], TAU_BWD, RMS_BWD,
                  what="window dv")


@pytest.mark.parametrize("window,d", [(0, 128), (40, 128), (0, 64)])
def test_autograd_function(gpu, window, d):
    """parallax_prefill_attention under torch autograd: the forward equals
    parallax_prefill, and loss.backward() gives exactly the C ABI backward's
    gradients (in the inputs' bf16) for the loss sum(dout * out); the oracle
    checks them too."""
    q, rho, k, v, dout, scale = case(2, 150, 4, 2, 61, gpu, d)
    leaves = [t.clone().requires_grad_(True) for t in (q, rho, k, v)]
    out = plx.parallax_prefill_attention(*leaves, scale=scale, window=window)
    (out * dout.float()).sum().backward()
    torch.cuda.synchronize()
    stats, grads = forward_backward(q, rho, k, v, dout, scale, window)
    assert torch.equal(out.detach(), stats[0])
    for leaf, g in zip(leaves, grads):
        assert leaf.grad.dtype == torch.bfloat16
        assert torch.equal(leaf.grad, g.to(torch.bfloat16))
    h = [host_array(t) for t in (q, rho, k, v, dout)]
    ref = oracle.prefill_backward(*h[:4], h[4], scale, window=window)
    for leaf, r, name in zip(leaves, ref, ("dq", "drho", "dk", "dv")):
        # one more bf16 rounding of the gradient itself: 2^-9 relative
        assert_parity(leaf.grad, r, TAU_BWD, RMS_BWD, what=f"autograd {name}")


def test_graph_replay(gpu):
    """Forward with statistics plus backward captured in one HIP graph
    replays to the eager result, with eager calls in between."""
    q, rho, k, v, dout, scale = case(1, 300, 4, 2, 18, gpu)
    stats, grads = forward_backward(q, rho, k, v, dout, scale)
    want = [t.clone() for t in grads]
    ws = torch.zeros(1 << 20, dtype=torch.uint8, device=gpu)
    outs = [torch.empty_like(t) for t in grads]
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        out, lse, rmean, o_sa = plx.parallax_prefill(q, rho, k, v, scale=scale, return_stats=True)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            # the forward again (its statistics are those of the eager call
            # above: same inputs), then the backward
            fo = plx.parallax_prefill(q, rho, k, v, scale=scale, out=out)
            plx.parallax_prefill_backward(q, rho, k, v, dout, fo, o_sa, lse, rmean, scale=scale,
                                          dq=outs[0], drho=outs[1], dk=outs[2], dv=outs[3],
                                          workspace=ws)
    other = case(1, 100, 2, 1, 19, gpu)
    for r in range(3):
        for t in outs:
            t.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        for a, b in zip(want, outs):
            assert torch.equal(a, b), f"replay {r}"
        forward_backward(*other[:5], other[5])


@pytest.mark.parametrize("scale", [0.0, -0.09, 0.4])
@pytest.mark.parametrize("d,W", [(128, 0), (64, 0), (128, 37)])
def test_any_finite_scale(gpu, scale, d, W):
    """The logit scale may be zero (uniform weights over each row's keys) or
    negative: every row of the forward, its statistics and the four
    gradients against the oracle at the same scale."""
    S, Hq, Hkv = 100, 4, 2
    q, rho, k, v, dout, _ = case(1, S, Hq, Hkv, 11, gpu, d)
    stats, grads = forward_backward(q, rho, k, v, dout, scale, window=W)
    what = f"scale={scale} d={d} W={W}"
    ref = oracle.prefill(*(host_array(t) for t in (q, rho, k, v)), scale, window=W)
    assert_parity(stats[0], ref, TAU_BF16, RMS_PREFILL, what=f"{what} out")
    check_stats(stats, q, rho, k, v, scale, window=W, what=what)
    ref = oracle.prefill_backward(*(host_array(t) for t in (q, rho, k, v, dout)), scale,
                                  window=W)
    for name, g, r in zip(("dq", "drho", "dk", "dv"), grads, ref):
        assert_parity(g, r, TAU_BWD, RMS_BWD, what=f"{what} {name}")
    if scale == 0.0:  # uniform weights: o_SA is the mean of the row's values, dq = 0
        vv = v.double()[0].cpu()
        for i in (0, 1, 36, 37, 99):
            lo = max(0, i - W + 1) if W else 0
            want = vv[lo:i + 1].mean(0)
            for h in range(Hq):
                got = stats[3][0, i, h].double().cpu()
                assert float((got - want[h // 2]).abs().max()) < 2e-2
        assert float(grads[0].abs().max()) == 0.0
