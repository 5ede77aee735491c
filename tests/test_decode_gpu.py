"""GPU parity of parallax_decode against the fp64 oracle (through the C ABI).

Cases follow the decode workloads: the tiny fp32 row (batch 1, one head,
d = 64, 128 tokens; also rho = 0 and a single token), the 1.7B-like GQA shape
(batch 8, 16 query / 8 KV heads, d = 128, 4096 tokens, bf16 cache), ragged
lengths around wave/page/split boundaries, empty rows, and the paged cache.
"""
import dataclasses
import math

import numpy as np
import pytest
import scipy.special
import torch

import oracle
import parallax_local_linear_decode_amd as plx
from parallax_local_linear_decode_amd.workloads import decode_inputs, host_array, paged_inputs

from helpers import (RMS_DECODE_BF16, TAU_BF16, TAU_F32, assert_parity, gather_sequences,
                     oracle_decode, parity)

pytestmark = pytest.mark.gpu


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


# ------------------------------------------------------------- tiny fp32 ---

def test_tiny_fp32(gpu):
    inp = to(decode_inputs(1, 1, 1, 64, 128, kv_dtype=torch.float32, seed=0), gpu)
    ref = oracle_decode(inp, form="explicit")
    assert_parity(run(inp), ref, TAU_F32, what="tiny fp32")


def test_tiny_fp32_rho_zero_is_softmax(gpu):
    inp = to(decode_inputs(1, 1, 1, 64, 128, kv_dtype=torch.float32, seed=0, rho_zero=True), gpu)
    q, k, v = (host_array(t).astype(np.float64) for t in (inp.q, inp.k, inp.v))
    want = scipy.special.softmax(inp.scale * (k[0, 0] @ q[0, 0])) @ v[0, 0]
    assert_parity(run(inp)[0, 0], want, TAU_F32, what="rho=0")


def test_tiny_fp32_single_token_is_value(gpu):
    inp = to(decode_inputs(1, 1, 1, 64, 1, kv_dtype=torch.float32, seed=0), gpu)
    assert_parity(run(inp)[0, 0], host_array(inp.v)[0, 0, 0], TAU_F32, what="ctx=1")


def test_tiny_fp32_lla_solved_probe(gpu):
    """With the solved probe rho* the output is the intercept of the
    softmax-weighted local linear fit (numpy lstsq), on the GPU too."""
    d, L = 64, 128
    inp = decode_inputs(1, 1, 1, d, L, kv_dtype=torch.float32, seed=3)
    q, K, V = (host_array(t).astype(np.float64) for t in (inp.q, inp.k, inp.v))
    q, K, V = q[0, 0], K[0, 0], V[0, 0]
    p = scipy.special.softmax(inp.scale * (K @ q))
    kbar = p @ K
    S_KK = ((K - kbar) * p[:, None]).T @ (K - kbar)
    rho_star = np.linalg.solve(S_KK, kbar - q)
    X = np.hstack([np.ones((L, 1)), K - q])
    w = np.sqrt(p)[:, None]
    coef, *_ = np.linalg.lstsq(X * w, V * w, rcond=None)
    inp.rho = torch.tensor(rho_star, dtype=torch.float32).reshape(1, 1, d)
    ref = oracle_decode(inp, form="explicit")[0, 0]
    inp = to(inp, gpu)
    out = run(inp)[0, 0]
    # the probe is rounded to fp32 on its way in; compare to the oracle on that
    # probe, and to the regression intercept at the size of that rounding
    assert_parity(out, ref, TAU_F32, what="solved probe vs oracle")
    assert np.max(np.abs(out.double().cpu().numpy() - coef[0])) < 1e-3


def test_tiny_fp32_invariants(gpu):
    inp = to(decode_inputs(2, 4, 2, 64, 77, kv_dtype=torch.float32, seed=4), gpu)
    base = run(inp).clone()
    c = torch.randn(64, device=gpu)
    shifted = decode_inputs(2, 4, 2, 64, 77, kv_dtype=torch.float32, seed=4)
    shifted = to(shifted, gpu)
    shifted.v = shifted.v + c
    assert (run(shifted) - (base + c)).abs().max().item() < 1e-4
    r2 = 0.1 * torch.randn_like(inp.rho)
    rho = inp.rho.clone()
    inp.rho = rho + r2
    o12 = run(inp).clone()
    inp.rho = torch.zeros_like(rho)
    o0 = run(inp).clone()
    inp.rho = r2
    o2 = run(inp).clone()
    assert (o12 + o0 - base - o2).abs().max().item() < 1e-5


# ------------------------------------------------------- 1.7B-like decode ---

@pytest.mark.parametrize("v_mode", ["iid", "correlated"])
def test_gqa_bf16_full_size(gpu, v_mode):
    inp = to(decode_inputs(8, 16, 8, 128, 4096, seed=0, v_mode=v_mode), gpu)
    ref = oracle_decode(inp)
    assert_parity(run(inp), ref, TAU_BF16, RMS_DECODE_BF16, what=f"1.7B-like {v_mode}")


def test_gqa_bf16_rho_zero_is_softmax(gpu):
    inp = to(decode_inputs(8, 16, 8, 128, 4096, seed=0, rho_zero=True), gpu)
    ref = oracle_decode(inp)
    assert_parity(run(inp), ref, TAU_BF16, RMS_DECODE_BF16, what="rho=0")


@pytest.mark.slow
@pytest.mark.parametrize("B,L", [(1024, 32768), (2048, 8192), (2048, 128), (1, 32768)])
def test_sweep_corners_sampled(gpu, B, L):
    """Corners of the batch x context sweep (16/8 heads, d 128, bf16 KV) in
    the launch configuration the bench times (the library's split choice):
    the largest cache (1024 x 32768 tokens, 137 GB), the most rows (2048 at
    8192 and at 128 tokens) and one long row.  Sampled sequences, including
    the first and last, against the oracle."""
    kv = B * 8 * L * 128 * 2 * 2
    if kv * 1.1 > torch.cuda.mem_get_info()[0]:
        pytest.skip(f"needs {kv / 1e9:.0f} GB of free HBM")
    inp = decode_inputs(B, 16, 8, 128, L, seed=B + L, device=gpu)
    out = run(inp)
    rng = np.random.default_rng(B + L)
    rows = sorted({0, B - 1, *(int(x) for x in rng.integers(0, B, 6))})
    sel = torch.as_tensor(rows, dtype=torch.long, device=gpu)
    sub = dataclasses.replace(inp, q=inp.q[sel], rho=inp.rho[sel], k=inp.k[sel], v=inp.v[sel])
    ref = oracle_decode(sub)
    got = out[sel]
    del inp, out, sub
    torch.cuda.empty_cache()
    assert_parity(got, ref, TAU_BF16, RMS_DECODE_BF16, what=f"sweep {B} x {L}")


# ------------------------------------------------------------------ edges ---

@pytest.mark.parametrize("kv_dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("G", [1, 2, 4, 8])
def test_ragged_lengths(gpu, kv_dtype, d, G):
    lens = [1, 2, 15, 16, 17, 31, 32, 33, 63, 64, 65, 127, 129, 200, 0, 257]
    B, Hkv, Lcap = len(lens), 2, 264
    inp = decode_inputs(B, Hkv * G, Hkv, d, Lcap, kv_dtype=kv_dtype, seed=G * 100 + d)
    inp.seq_lens = torch.tensor(lens, dtype=torch.int32)
    for b, L in enumerate(lens):  # tokens past seq_lens must never be read
        inp.k[b, :, L:] = float("nan")
        inp.v[b, :, L:] = float("nan")
    ref = oracle_decode(inp)
    inp = to(inp, gpu)
    tau = TAU_F32 if kv_dtype == torch.float32 else TAU_BF16
    for split in (0, 256):
        out = run(inp, split_tokens=split)
        assert_parity(out, ref, tau, None if kv_dtype == torch.float32 else RMS_DECODE_BF16,
                      what=f"ragged split={split}")
        assert torch.all(out[lens.index(0)] == 0)


@pytest.mark.parametrize("kv_dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("G", [1, 2, 4, 8])
def test_many_splits(gpu, kv_dtype, d, G):
    """Rows of up to 36 splits of 256 tokens: above sixteen splits the last
    arriving split merges the records in several ranges side by side when
    the workgroup has threads to spare (G * d below its thread count), else
    in one range; rows of 17, 16, 2, 1 and 0 splits beside them."""
    lens = [9000, 4300, 4096, 300, 0, 8193]
    B, Hkv, Lcap = len(lens), 2, 9000
    inp = decode_inputs(B, Hkv * G, Hkv, d, Lcap, kv_dtype=kv_dtype, seed=G * 7 + d)
    inp.seq_lens = torch.tensor(lens, dtype=torch.int32)
    for b, L in enumerate(lens):
        inp.k[b, :, L:] = float("nan")
        inp.v[b, :, L:] = float("nan")
    ref = oracle_decode(inp)
    inp = to(inp, gpu)
    tau = TAU_F32 if kv_dtype == torch.float32 else TAU_BF16
    out = run(inp, split_tokens=256)
    assert_parity(out, ref, tau, None if kv_dtype == torch.float32 else RMS_DECODE_BF16,
                  what=f"many splits G={G} d={d}")
    assert torch.all(out[lens.index(0)] == 0)
    assert torch.equal(run(inp, split_tokens=256), out)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("G", [1, 2, 4, 8])
def test_short_rows(gpu, d, G):
    """A cache of at most 128 tokens gives workgroups of at most four 32-token
    steps, which run with four waves; ragged lengths, NaN past each."""
    lens = [1, 2, 15, 16, 17, 31, 32, 33, 63, 64, 65, 96, 127, 128, 0, 100]
    B, Hkv, Lcap = len(lens), 2, 128
    inp = decode_inputs(B, Hkv * G, Hkv, d, Lcap, seed=G * 10 + d)
    inp.seq_lens = torch.tensor(lens, dtype=torch.int32)
    for b, L in enumerate(lens):
        inp.k[b, :, L:] = float("nan")
        inp.v[b, :, L:] = float("nan")
    ref = oracle_decode(inp)
    inp = to(inp, gpu)
    out = run(inp)
    assert_parity(out, ref, TAU_BF16, RMS_DECODE_BF16, what=f"short rows G={G} d={d}")
    assert torch.all(out[lens.index(0)] == 0)


def test_split_choices_agree(gpu):
    inp = to(decode_inputs(3, 16, 8, 128, 3000, seed=7), gpu)
    ref = oracle_decode(inp)
    outs = []
    for split in (256, 512, 768, 1024, 2048, 3072):
        out = run(inp, split_tokens=split).clone()
        assert_parity(out, ref, TAU_BF16, RMS_DECODE_BF16, what=f"split={split}")
        outs.append(out)
    for o in outs[1:]:
        assert (o - outs[0]).abs().max().item() < 1e-5


def test_deterministic(gpu):
    inp = to(decode_inputs(4, 16, 8, 128, 2500, seed=8), gpu)
    first = run(inp).clone()
    for _ in range(20):
        assert torch.equal(run(inp), first)


@pytest.mark.slow
def test_full_size_deterministic(gpu):
    """Batch 8, 16/8 heads, 4096 and 32768 tokens: repeated launches (split
    kernel plus merge) return identical bits under a full-chip load."""
    for L in (4096, 32768):
        inp = decode_inputs(8, 16, 8, 128, L, seed=9, device=gpu)
        first = run(inp).clone()
        for i in range(50):
            assert torch.equal(run(inp), first), f"L={L} launch {i} differs"


def test_workspace_reuse_across_shapes(gpu):
    """One workspace, filled with garbage first, serves calls of different
    shapes back to back (its contents on entry never matter)."""
    ws = torch.randint(0, 256, (1 << 24,), dtype=torch.uint8, device=gpu)
    for i, (B, L) in enumerate([(2, 700), (8, 4096), (2, 700), (12, 3000), (5, 1500)]):
        inp = to(decode_inputs(B, 16, 8, 128, L, seed=20 + i), gpu)
        out = run(inp, workspace=ws)
        assert_parity(out, oracle_decode(inp), TAU_BF16, RMS_DECODE_BF16, what=f"reuse {i}")


def test_side_stream_calls_grow_their_workspace(gpu):
    """Calls on a side stream, each larger than the last, so the binding's
    per-stream workspace grows while earlier launches may still be queued:
    the same bits as the same calls on the default stream."""
    shapes = [(1, 300), (4, 2000), (8, 4096), (16, 8192)]
    inps = [to(decode_inputs(B, 16, 8, 128, L, seed=30 + i), gpu) for i, (B, L) in enumerate(shapes)]
    want = [run(inp).clone() for inp in inps]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        got = [plx.parallax_decode(inp.q, inp.rho, inp.k, inp.v, scale=inp.scale) for inp in inps]
    torch.cuda.synchronize()
    for i, (w, g) in enumerate(zip(want, got)):
        assert torch.equal(w, g), f"shape {shapes[i]}"


def test_graph_replay(gpu):
    """A captured decode replays correctly several times, with eager calls on
    the same workspace in between."""
    inp = to(decode_inputs(4, 16, 8, 128, 2000, seed=30), gpu)
    ref = oracle_decode(inp)
    ws = torch.zeros(1 << 22, dtype=torch.uint8, device=gpu)
    out = torch.empty((4, 16, 128), dtype=torch.float32, device=gpu)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        run(inp, workspace=ws, out=out)  # warm up on the capture stream
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            plx.parallax_decode(inp.q, inp.rho, inp.k, inp.v, scale=inp.scale, out=out,
                                workspace=ws)
    other = to(decode_inputs(2, 16, 8, 128, 900, seed=31), gpu)
    for r in range(4):
        out.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert_parity(out, ref, TAU_BF16, RMS_DECODE_BF16, what=f"replay {r}")
        run(other, workspace=ws)  # an eager call of another shape in between


# ------------------------------------------------------------------ paged ---

def test_paged_small(gpu):
    inp = paged_inputs(12, 16, 8, 128, ctx_lo=1, ctx_hi=700, seed=0, rho_zero_rows=3)
    ref = oracle_decode(inp)
    inp = to(inp, gpu)
    for split in (0, 256, 512):
        assert_parity(run(inp, split_tokens=split), ref, TAU_BF16, RMS_DECODE_BF16,
                      what=f"paged split={split}")


def test_paged_short_rows(gpu):
    """Paged rows of 1-128 tokens (the four-wave workgroups), NaN-poisoned
    tails and unused block-table entries, rho = 0 for two rows."""
    inp = paged_inputs(24, 16, 8, 128, ctx_lo=1, ctx_hi=128, seed=3, rho_zero_rows=2)
    ref = oracle_decode(inp)
    inp = to(inp, gpu)
    assert_parity(run(inp), ref, TAU_BF16, RMS_DECODE_BF16, what="paged short rows")


def test_paged_equals_contiguous(gpu):
    """The same logical sequences through the page table and laid out
    contiguously give the same result (same split => same reduction order)."""
    inp = paged_inputs(4, 16, 8, 128, seq_lens=[100, 1024, 777, 2048], seed=1)
    B, P = 4, 16
    lens = inp.seq_lens.tolist()
    Lcap = max(lens)
    kc = torch.zeros((B, 8, Lcap, 128), dtype=torch.bfloat16)
    vc = torch.zeros_like(kc)
    for b in range(B):
        j = torch.arange(lens[b])
        pg = inp.block_table[b, j // P].long()
        kc[b, :, :lens[b]] = inp.k[pg, :, j % P].transpose(0, 1)
        vc[b, :, :lens[b]] = inp.v[pg, :, j % P].transpose(0, 1)
    inp = to(inp, gpu)
    op = run(inp, split_tokens=256).clone()
    oc = plx.parallax_decode(inp.q, inp.rho, kc.to(gpu), vc.to(gpu), scale=inp.scale,
                             seq_lens=inp.seq_lens, split_tokens=256)
    torch.cuda.synchronize()
    assert torch.equal(op, oc)


@pytest.mark.slow
def test_paged_full_size_sampled(gpu):
    """Paged workload at full size: 256 sequences, lengths U[128, 32768],
    shuffled 16-token pages, NaN-poisoned tails, rho = 0 for sequences 0-31.
    Every output is checked for finiteness; sampled sequences (the rho = 0
    ones, the longest, the shortest and random ones) against the oracle."""
    inp = paged_inputs(256, 16, 8, 128, seed=0, rho_zero_rows=32, device=gpu)
    out = run(inp)
    assert torch.isfinite(out).all()
    lens = inp.seq_lens.cpu().numpy()
    rng = np.random.default_rng(0)
    pick = sorted(set([0, 1, 2, 31, int(np.argmax(lens)), int(np.argmin(lens))] +
                      list(rng.choice(np.arange(32, 256), 10, replace=False))))
    q, rho, k, v, sl, table = gather_sequences(inp, pick)
    ref = oracle.decode(q, rho, k, v, inp.scale, seq_lens=sl, block_table=table)
    assert_parity(out[pick], ref, TAU_BF16, RMS_DECODE_BF16, what="paged full")


def test_graph_capture_needs_an_explicit_workspace(gpu):
    """Under capture the binding does not hand out its cached per-stream
    workspace (growing it would synchronise, and graphs captured on one
    stream would share it): a call without workspace= raises, one with it is
    captured and replays correctly."""
    inp = to(decode_inputs(4, 16, 8, 128, 2000, seed=32), gpu)
    ref = oracle_decode(inp)
    s = torch.cuda.Stream()
    out = torch.empty((4, 16, 128), dtype=torch.float32, device=gpu)
    with torch.cuda.stream(s):
        run(inp, out=out)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            try:  # refused on the host, before any HIP call
                plx.parallax_decode(inp.q, inp.rho, inp.k, inp.v, scale=inp.scale, out=out)
                refused = ""
            except RuntimeError as e:
                refused = str(e)
            out.zero_()
    torch.cuda.synchronize()
    assert "workspace" in refused
    ws = torch.zeros(1 << 22, dtype=torch.uint8, device=gpu)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            plx.parallax_decode(inp.q, inp.rho, inp.k, inp.v, scale=inp.scale, out=out,
                                workspace=ws)
    for r in range(3):
        out.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert_parity(out, ref, TAU_BF16, RMS_DECODE_BF16, what=f"replay {r}")


def test_concurrent_calls_on_two_streams(gpu):
    """Two decodes with their own workspaces running at the same time on two
    streams (their splits' merges in flight together, rows of different
    lengths and split counts) return the bits of the same calls run one
    after the other; repeated a few times."""
    a = to(decode_inputs(8, 16, 8, 128, 4096, seed=40), gpu)
    b = to(decode_inputs(2, 16, 8, 128, 20000, seed=41), gpu)
    want_a, want_b = run(a).clone(), run(b).clone()
    wa = torch.randint(0, 256, (1 << 22,), dtype=torch.uint8, device=gpu)
    wb = torch.randint(0, 256, (1 << 22,), dtype=torch.uint8, device=gpu)
    sa, sb = torch.cuda.Stream(), torch.cuda.Stream()
    for i in range(5):
        sa.wait_stream(torch.cuda.current_stream())
        sb.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(sa):
            oa = plx.parallax_decode(a.q, a.rho, a.k, a.v, scale=a.scale, workspace=wa)
        with torch.cuda.stream(sb):
            ob = plx.parallax_decode(b.q, b.rho, b.k, b.v, scale=b.scale, workspace=wb)
        torch.cuda.synchronize()
        assert torch.equal(oa, want_a), f"round {i}: stream a"
        assert torch.equal(ob, want_b), f"round {i}: stream b"
