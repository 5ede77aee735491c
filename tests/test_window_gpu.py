"""GPU parity of the local-window variant (keys of a row limited to its W
most recent ones; the local window the Parallax page leaves open, section
3.1) against the fp64 oracle, through the C ABI.  Tokens outside each row's
window hold NaN in the decode tests, so any read of them shows."""
import numpy as np
import pytest
import torch

import oracle
import parallax_local_linear_decode_amd as plx
from parallax_local_linear_decode_amd.workloads import (decode_inputs, host_array, paged_inputs,
                                                        prefill_inputs)

from helpers import (RMS_DECODE_BF16, RMS_PREFILL, TAU_BF16, TAU_F32, assert_parity,
                     oracle_decode)

pytestmark = pytest.mark.gpu

WINDOWS = [1, 5, 31, 32, 33, 100, 300]


def to(inp, dev):
    for name in ("q", "rho", "k", "v", "seq_lens", "block_table"):
        t = getattr(inp, name)
        if t is not None:
            setattr(inp, name, t.to(dev))
    return inp


def run(inp, **kw):
    out = plx.parallax_decode(inp.q, inp.rho, inp.k, inp.v, scale=inp.scale,
                              seq_lens=inp.seq_lens, block_table=inp.block_table, **kw)
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("kv_dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("G", [1, 2, 4, 8])
def test_window_decode(gpu, kv_dtype, d, G):
    lens = [0, 1, 2, 31, 32, 33, 47, 64, 100, 129, 200, 257, 300, 301, 520, 700]
    B, Hkv, Lcap = len(lens), 2, 704
    inp = decode_inputs(B, Hkv * G, Hkv, d, Lcap, kv_dtype=kv_dtype, seed=G * 7 + d)
    inp.seq_lens = torch.tensor(lens, dtype=torch.int32)
    k0, v0 = inp.k.clone(), inp.v.clone()
    tau = TAU_F32 if kv_dtype == torch.float32 else TAU_BF16
    rms = None if kv_dtype == torch.float32 else RMS_DECODE_BF16
    dev_lens = inp.seq_lens.to(gpu)
    for W in WINDOWS:
        inp.k, inp.v = k0.clone(), v0.clone()
        for b, L in enumerate(lens):  # NaN outside each row's window
            inp.k[b, :, L:] = float("nan")
            inp.v[b, :, L:] = float("nan")
            inp.k[b, :, :max(0, L - W)] = float("nan")
            inp.v[b, :, :max(0, L - W)] = float("nan")
        ref = oracle.decode(host_array(inp.q), host_array(inp.rho), host_array(inp.k),
                            host_array(inp.v), inp.scale, seq_lens=host_array(inp.seq_lens),
                            window=W)
        q, rho, k, v = (t.to(gpu) for t in (inp.q, inp.rho, inp.k, inp.v))
        for split in (0, 256):
            out = plx.parallax_decode(q, rho, k, v, scale=inp.scale, seq_lens=dev_lens,
                                      split_tokens=split, window=W)
            torch.cuda.synchronize()
            assert_parity(out, ref, tau, rms, what=f"window={W} split={split}")
            assert torch.all(out[lens.index(0)] == 0)


def test_window_decode_long_rows_many_splits(gpu):
    """Rows of 20000 tokens, window 5000 (several splits per row, the window
    start inside a split), and a window at least the row (full attention)."""
    inp = decode_inputs(2, 16, 8, 128, 20000, seed=41)
    ref5k = oracle_decode(inp, window=5000)
    inp = to(inp, gpu)
    for split in (0, 1024):
        assert_parity(run(inp, window=5000, split_tokens=split), ref5k, TAU_BF16,
                      RMS_DECODE_BF16, what=f"window 5000 split={split}")
    assert torch.equal(run(inp, window=20000), run(inp))


@pytest.mark.parametrize("kv_dtype", [torch.bfloat16, torch.float32])
def test_window_paged(gpu, kv_dtype):
    """Paged cache: block-table entries of pages that hold only tokens before
    the window point at the NaN page, and pre-window slots of the window's
    first page are NaN too."""
    inp = paged_inputs(20, 16, 8, 128, ctx_lo=1, ctx_hi=1500, seed=42, rho_zero_rows=2,
                       kv_dtype=kv_dtype)
    tau = TAU_F32 if kv_dtype == torch.float32 else TAU_BF16
    rms = None if kv_dtype == torch.float32 else RMS_DECODE_BF16
    NB = inp.k.shape[0] - 1  # the all-NaN page
    for W in (1, 17, 100, 1000):
        table = inp.block_table.clone()
        k, v = inp.k.clone(), inp.v.clone()
        for b in range(table.shape[0]):
            L = int(inp.seq_lens[b])
            tb = max(0, L - W)
            table[b, :tb // 16] = NB
            if tb % 16:
                pg = int(inp.block_table[b, tb // 16])
                k[pg, :, :tb % 16] = float("nan")
                v[pg, :, :tb % 16] = float("nan")
        ref = oracle.decode(host_array(inp.q), host_array(inp.rho), host_array(k), host_array(v),
                            inp.scale, seq_lens=host_array(inp.seq_lens),
                            block_table=host_array(table), window=W)
        out = plx.parallax_decode(inp.q.to(gpu), inp.rho.to(gpu), k.to(gpu), v.to(gpu),
                                  scale=inp.scale, seq_lens=inp.seq_lens.to(gpu),
                                  block_table=table.to(gpu), window=W)
        torch.cuda.synchronize()
        assert_parity(out, ref, tau, rms, what=f"paged window={W}")


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("S", [1, 33, 100, 300])
@pytest.mark.parametrize("Hq,Hkv", [(2, 1), (4, 2), (8, 2), (16, 2)])
def test_window_prefill(gpu, S, Hq, Hkv, d):
    q, rho, k, v, scale = prefill_inputs(2, S, Hq, Hkv, d, seed=S + Hq + d)
    hq, hr, hk, hv = (host_array(t) for t in (q, rho, k, v))
    dq, dr, dk, dv = (t.to(gpu) for t in (q, rho, k, v))
    for W in [1, 5, 31, 32, 33, 64, 100]:
        ref = oracle.prefill(hq, hr, hk, hv, scale, window=W)
        out = plx.parallax_prefill(dq, dr, dk, dv, scale=scale, window=W)
        torch.cuda.synchronize()
        assert_parity(out, ref, TAU_BF16, RMS_PREFILL, what=f"prefill S={S} window={W}")


def test_window_prefill_at_least_the_sequence_is_full(gpu):
    q, rho, k, v, scale = (t.to(gpu) if isinstance(t, torch.Tensor) else t
                           for t in prefill_inputs(1, 300, 4, 2, 128, seed=43))
    full = plx.parallax_prefill(q, rho, k, v, scale=scale).clone()
    for W in (300, 301, 5000):
        assert torch.equal(plx.parallax_prefill(q, rho, k, v, scale=scale, window=W), full)


@pytest.mark.slow
def test_window_prefill_full_size_sampled_rows(gpu):
    """Batch 4 x 8192 tokens, 16/8 heads, window 1024: rows around the window
    and tile edges plus random rows, for every (batch, head)."""
    B, S, Hq, Hkv, W = 4, 8192, 16, 8, 1024
    q, rho, k, v, scale = prefill_inputs(B, S, Hq, Hkv, 128, seed=44, device=gpu)
    out = plx.parallax_prefill(q, rho, k, v, scale=scale, window=W)
    torch.cuda.synchronize()
    assert torch.isfinite(out).all()
    rng = np.random.default_rng(44)
    rows = sorted(set([0, 1, 31, 32, 1022, 1023, 1024, 1025, 1056, 4095, 4096, 8191] +
                      list(rng.integers(0, S, 24))))
    ref = oracle.prefill(*(host_array(t) for t in (q, rho, k, v)), scale,
                         rows=np.array(rows, dtype=np.int32), window=W)
    assert_parity(out[:, rows], ref, TAU_BF16, RMS_PREFILL, what="prefill window full size")
