"""GPU parity of parallax_prefill (causal, bf16 matrix cores) against the
fp64 oracle, through the C ABI.

Small cases compare every row (ragged sequence lengths around the 32-key
tile and 64-row block edges, GQA groups 1/2/4); the full-size workload
(batch 4, 8192 tokens, 16 query / 8 KV heads, d = 128) compares sampled rows.
"""
import numpy as np
import pytest
import scipy.special
import torch

import oracle
import parallax_local_linear_decode_amd as plx
from parallax_local_linear_decode_amd.workloads import host_array, prefill_inputs

from helpers import RMS_PREFILL, TAU_BF16, assert_parity

pytestmark = pytest.mark.gpu


def run(q, rho, k, v, scale):
    out = plx.parallax_prefill(q, rho, k, v, scale=scale)
    torch.cuda.synchronize()
    return out


def host(*ts):
    return [host_array(t) for t in ts]


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("S", [1, 17, 31, 32, 33, 64, 100, 257])
@pytest.mark.parametrize("Hq,Hkv", [(2, 1), (4, 2), (2, 2), (8, 2), (8, 1), (16, 2), (16, 1)])
def test_small_all_rows(gpu, S, Hq, Hkv, d):
    q, rho, k, v, scale = prefill_inputs(2, S, Hq, Hkv, d, seed=S * 10 + Hq + d)
    ref = oracle.prefill(*host(q, rho, k, v), scale)
    out = run(*(t.to(gpu) for t in (q, rho, k, v)), scale)
    assert_parity(out, ref, TAU_BF16, RMS_PREFILL, what=f"d={d} S={S} {Hq}/{Hkv}")


def test_head_dim_64_larger(gpu):
    """d = 64 over several query blocks and K/V tiles (1000 tokens, 16/8
    heads), every row, plus the rho = 0 softmax case."""
    q, rho, k, v, scale = prefill_inputs(2, 1000, 16, 8, 64, seed=64)
    ref = oracle.prefill(*host(q, rho, k, v), scale)
    out = run(*(t.to(gpu) for t in (q, rho, k, v)), scale)
    assert_parity(out, ref, TAU_BF16, RMS_PREFILL, what="d=64 S=1000")
    zero = torch.zeros_like(rho)
    ref0 = oracle.prefill(*host(q, zero, k, v), scale)
    out0 = run(*(t.to(gpu) for t in (q, zero, k, v)), scale)
    assert_parity(out0, ref0, TAU_BF16, RMS_PREFILL, what="d=64 rho=0")


def test_first_row_is_first_value(gpu):
    q, rho, k, v, scale = prefill_inputs(2, 70, 4, 2, 128, seed=5)
    out = run(*(t.to(gpu) for t in (q, rho, k, v)), scale)
    vv = v.float()
    for h in range(4):
        assert (out[:, 0, h].cpu() - vv[:, 0, h // 2]).abs().max().item() < 1e-5


def test_rho_zero_is_causal_softmax(gpu):
    q, rho, k, v, scale = prefill_inputs(1, 150, 2, 1, 128, seed=6)
    rho = torch.zeros_like(rho)
    out = run(*(t.to(gpu) for t in (q, rho, k, v)), scale)
    qq, kk, vv = (t.double().numpy()[0] for t in (q, k, v))
    S = 150
    mask = np.tril(np.ones((S, S), dtype=bool))
    for h in range(2):
        logits = scale * qq[:, h] @ kk[:, 0].T
        p = scipy.special.softmax(np.where(mask, logits, -np.inf), axis=1)
        assert_parity(out[0, :, h], p @ vv[:, 0], TAU_BF16, RMS_PREFILL, what=f"rho=0 h={h}")


def test_correlated_values(gpu):
    """V = K M^T + noise makes the covariance branch large; every row checked."""
    q, rho, k, v, scale = prefill_inputs(1, 300, 4, 2, 128, seed=7)
    g = torch.Generator().manual_seed(8)
    M = torch.randn(128, 128, generator=g) / 128 ** 0.5
    v = (k.float() @ M.T + 0.1 * torch.randn(k.shape, generator=g)).to(torch.bfloat16)
    rho = (3.0 * rho.float()).to(torch.bfloat16)
    ref = oracle.prefill(*host(q, rho, k, v), scale)
    out = run(*(t.to(gpu) for t in (q, rho, k, v)), scale)
    assert_parity(out, ref, TAU_BF16, RMS_PREFILL, what="correlated")


def test_deterministic(gpu):
    q, rho, k, v, scale = (t.to(gpu) if isinstance(t, torch.Tensor) else t
                           for t in prefill_inputs(2, 500, 4, 2, 128, seed=9))
    first = run(q, rho, k, v, scale).clone()
    for _ in range(5):
        assert torch.equal(run(q, rho, k, v, scale), first)


@pytest.mark.slow
def test_full_size_sampled_rows(gpu):
    """Batch 4, 8192 tokens, 16/8 heads, d = 128: rows at the tile, block and
    sequence edges plus 32 random rows, for every (batch, head)."""
    B, S, Hq, Hkv = 4, 8192, 16, 8
    q, rho, k, v, scale = prefill_inputs(B, S, Hq, Hkv, 128, seed=0, device=gpu)
    out = run(q, rho, k, v, scale)
    assert torch.isfinite(out).all()
    rng = np.random.default_rng(0)
    rows = sorted(set([0, 1, 2, 31, 32, 63, 64, 65, 127, 128, 129, 4095, 4096, 8190, 8191] +
                      list(rng.integers(0, S, 32))))
    ref = oracle.prefill(*host(q, rho, k, v), scale, rows=np.array(rows, dtype=np.int32))
    assert_parity(out[:, rows], ref, TAU_BF16, RMS_PREFILL, what="prefill full size")


@pytest.mark.slow
def test_long_sequence_sampled_rows(gpu):
    """One sequence of 32768 tokens (16/8 heads, d 128): rows at tile and
    block edges, the last rows and random rows, against the oracle."""
    B, S, Hq, Hkv = 1, 32768, 16, 8
    q, rho, k, v, scale = prefill_inputs(B, S, Hq, Hkv, 128, seed=21, device=gpu)
    out = run(q, rho, k, v, scale)
    rng = np.random.default_rng(21)
    rows = sorted(set([0, 127, 128, 16383, 16384, 32640, 32767] + list(rng.integers(0, S, 9))))
    ref = oracle.prefill(*host(q, rho, k, v), scale, rows=np.array(rows, dtype=np.int32))
    assert_parity(out[:, rows], ref, TAU_BF16, RMS_PREFILL, what="prefill 32768 tokens")


@pytest.mark.slow
def test_full_size_deterministic(gpu):
    """Repeated launches at batch 4 x 8192 tokens return identical bits: the
    K/V tiles and the score-to-value hand-off in LDS are race-free under a
    full-chip load, where timing differs from launch to launch."""
    B, S, Hq, Hkv = 4, 8192, 16, 8
    q, rho, k, v, scale = prefill_inputs(B, S, Hq, Hkv, 128, seed=3, device=gpu)
    first = run(q, rho, k, v, scale).clone()
    out = torch.empty_like(first)
    for i in range(20):
        out.fill_(float("nan"))
        plx.parallax_prefill(q, rho, k, v, scale=scale, out=out)
        torch.cuda.synchronize()
        assert torch.equal(out, first), f"launch {i} differs"


def test_strided_views_equal_contiguous(gpu):
    """q and rho as the two halves of one [B, S, 2, Hq, d] buffer (the layout
    the stacked projection writes), k and v as halves of [B, S, 2, Hkv, d],
    and out written into a wider buffer: the same bits as contiguous tensors."""
    B, S, Hq, Hkv, d = 2, 300, 4, 2, 128
    q, rho, k, v, scale = (t.to(gpu) if isinstance(t, torch.Tensor) else t
                           for t in prefill_inputs(B, S, Hq, Hkv, d, seed=9))
    want = run(q, rho, k, v, scale).clone()
    qr = torch.stack([q, rho], dim=2)          # [B, S, 2, Hq, d]
    kv = torch.stack([k, v], dim=2)            # [B, S, 2, Hkv, d]
    wide = torch.full((B, S, Hq, 2 * d), float("nan"), dtype=torch.float32, device=gpu)
    out = plx.parallax_prefill(qr[:, :, 0], qr[:, :, 1], kv[:, :, 0], kv[:, :, 1], scale=scale,
                               out=wide[..., d:])
    torch.cuda.synchronize()
    assert torch.equal(out, want)
    assert torch.isnan(wide[..., :d]).all()


@pytest.mark.parametrize("S,Hq,Hkv,window", [
    (33, 2, 2, 0), (257, 4, 2, 0), (257, 16, 2, 0), (600, 2, 1, 0), (600, 4, 1, 100),
    (100, 8, 2, 40), (500, 16, 1, 0)])
def test_workgroup_counts_agree(gpu, S, Hq, Hkv, window):
    """Head dim 128 runs a fixed set of persistent workgroups, each taking its
    share of the (query block, head block) items in turn (the next item's
    tiles and q / rho loaded during the current one's last positions), and
    the shortest items one per workgroup.  One persistent workgroup for
    almost every item, counts that are and are not multiples of 8 and the
    default give the same bits (outputs and the backward's statistics); every
    row of the one-workgroup run matches the oracle."""
    q, rho, k, v, scale = prefill_inputs(2, S, Hq, Hkv, 128, seed=S + Hq + window)
    ref = oracle.prefill(*host(q, rho, k, v), scale, window=window)
    dev = [t.to(gpu) for t in (q, rho, k, v)]
    runs = {}
    for wgs in (1, 3, 8, 16, 0):
        plain = plx.parallax_prefill(*dev, scale=scale, window=window, workgroups=wgs)
        stats = plx.parallax_prefill(*dev, scale=scale, window=window, workgroups=wgs,
                                     return_stats=True)
        torch.cuda.synchronize()
        assert torch.equal(plain, stats[0]), f"workgroups={wgs}: stats build differs"
        runs[wgs] = stats
    for wgs, got in runs.items():
        for name, a, b in zip(("out", "lse", "rmean", "o_sa"), got, runs[0]):
            assert torch.equal(a, b), f"workgroups={wgs}: {name} differs from the default"
    assert_parity(runs[1][0], ref, TAU_BF16, RMS_PREFILL, what=f"one workgroup S={S} W={window}")


def test_workgroups_ignored_at_head_dim_64(gpu):
    q, rho, k, v, scale = (t.to(gpu) if isinstance(t, torch.Tensor) else t
                           for t in prefill_inputs(2, 300, 8, 2, 64, seed=11))
    a = plx.parallax_prefill(q, rho, k, v, scale=scale, workgroups=1)
    b = plx.parallax_prefill(q, rho, k, v, scale=scale)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


@pytest.mark.slow
def test_full_size_few_workgroups_agree(gpu):
    """Batch 4 x 8192 (16/8 heads): the default one workgroup per CU, and 40
    workgroups (about a hundred items each), give identical bits, window or
    not."""
    B, S, Hq, Hkv = 4, 8192, 16, 8
    q, rho, k, v, scale = prefill_inputs(B, S, Hq, Hkv, 128, seed=13, device=gpu)
    for window in (0, 1024):
        a = plx.parallax_prefill(q, rho, k, v, scale=scale, window=window)
        b = plx.parallax_prefill(q, rho, k, v, scale=scale, window=window, workgroups=40)
        torch.cuda.synchronize()
        assert torch.equal(a, b), f"window {window}"
