"""parallax_decode_no_alloc (the decode entry point that allocates nothing;
its split partials live in the library's per-device scratch) against
parallax_decode and the oracle, through the C ABI."""
import dataclasses

import numpy as np
import pytest
import torch

import parallax_local_linear_decode_amd as plx
from parallax_local_linear_decode_amd.workloads import decode_inputs, paged_inputs

from helpers import RMS_DECODE_BF16, TAU_BF16, TAU_F32, assert_parity, oracle_decode

pytestmark = pytest.mark.gpu


def both(inp, **kw):
    """(parallax_decode with its own workspace, parallax_decode_no_alloc)."""
    want = plx.parallax_decode(inp.q, inp.rho, inp.k, inp.v, scale=inp.scale,
                               seq_lens=inp.seq_lens, block_table=inp.block_table, **kw)
    out = torch.full_like(want, float("nan"))
    got = plx.parallax_decode_no_alloc(inp.q, inp.rho, inp.k, inp.v, out, scale=inp.scale,
                                       seq_lens=inp.seq_lens, block_table=inp.block_table, **kw)
    torch.cuda.synchronize()
    assert got is out
    return want, got


def test_two_calls_second_smaller(gpu):
    """Batch 8 x 4096 (16/8 heads, four splits per row), then batch 3 x 1500
    on the same scratch: bitwise the workspace entry point's results, and
    within the oracle bounds."""
    for B, L, seed in ((8, 4096, 0), (3, 1500, 1)):
        inp = decode_inputs(B, 16, 8, 128, L, seed=seed, device=gpu)
        want, got = both(inp)
        assert torch.equal(got, want), f"batch {B} x {L}"
        assert_parity(got, oracle_decode(inp), TAU_BF16, RMS_DECODE_BF16, what=f"{B} x {L}")


def test_ragged_paged_fp32_and_window(gpu):
    """Paged ragged rows, an fp32 cache with explicit splits, and a window,
    back to back on the one scratch."""
    inp = paged_inputs(12, 16, 8, 128, ctx_lo=1, ctx_hi=900, seed=2, rho_zero_rows=2,
                       device=gpu)
    want, got = both(inp, split_tokens=256)
    assert torch.equal(got, want)
    assert_parity(got, oracle_decode(inp), TAU_BF16, RMS_DECODE_BF16, what="paged")
    inp = decode_inputs(4, 8, 2, 64, 700, kv_dtype=torch.float32, seed=3, device=gpu)
    inp.seq_lens = torch.tensor([700, 1, 0, 513], dtype=torch.int32, device=gpu)
    want, got = both(inp, split_tokens=256)
    assert torch.equal(got, want)
    assert_parity(got, oracle_decode(inp), TAU_F32, what="fp32 ragged")
    inp = decode_inputs(2, 16, 8, 128, 5000, seed=4, device=gpu)
    want, got = both(inp, window=1200)
    assert torch.equal(got, want)
    assert_parity(got, oracle_decode(inp, window=1200), TAU_BF16, RMS_DECODE_BF16, what="window")


def test_partials_beyond_the_scratch_take_longer_splits(gpu):
    """256 sequences x 16384 tokens, 64 query / 8 KV heads: the library's split
    choice would need 68 MB of partials, more than the scratch holds, so the
    call takes fewer, longer splits -- within the oracle bounds on sampled
    sequences and within fp32 rounding of the workspace entry point."""
    B, Hq, Hkv, d, L = 256, 64, 8, 128, 16384
    if B * Hkv * L * d * 4 * 1.2 > torch.cuda.mem_get_info()[0]:
        pytest.skip("needs 21 GB of free HBM")
    inp = decode_inputs(B, Hq, Hkv, d, L, seed=5, device=gpu)
    need = plx.parallax_decode_workspace_size(inp.q, inp.rho, inp.k, inp.v, scale=inp.scale)
    assert need > plx.NO_ALLOC_SCRATCH_BYTES
    want, got = both(inp)
    assert_parity(got, want.double().cpu().numpy(), 1e-5, 1e-5, what="vs workspace entry point")
    rows = [0, 77, 255]
    sel = torch.as_tensor(rows, dtype=torch.long, device=gpu)
    sub = dataclasses.replace(inp, q=inp.q[sel], rho=inp.rho[sel], k=inp.k[sel], v=inp.v[sel])
    ref = oracle_decode(sub)
    got = got[sel]
    del inp, sub, want
    torch.cuda.empty_cache()
    assert_parity(got, ref, TAU_BF16, RMS_DECODE_BF16, what="sampled vs oracle")


def test_out_must_be_given(gpu):
    inp = decode_inputs(1, 2, 1, 64, 10, seed=6, device=gpu)
    with pytest.raises(TypeError):
        plx.parallax_decode_no_alloc(inp.q, inp.rho, inp.k, inp.v, scale=inp.scale)


def test_captured_graph_replays(gpu):
    """The entry point under HIP graph capture (no workspace to bring): three
    replays, with eager calls of another shape on the same scratch between
    them, each checked against the workspace entry point's result."""
    inp = decode_inputs(4, 16, 8, 128, 3000, seed=7, device=gpu)
    other = decode_inputs(2, 16, 8, 128, 900, seed=8, device=gpu)
    want, _ = both(inp)
    out = torch.empty_like(want)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        plx.parallax_decode_no_alloc(inp.q, inp.rho, inp.k, inp.v, out, scale=inp.scale)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            plx.parallax_decode_no_alloc(inp.q, inp.rho, inp.k, inp.v, out, scale=inp.scale)
    torch.cuda.synchronize()
    o2 = torch.empty((2, 16, 128), dtype=torch.float32, device=gpu)
    for r in range(3):
        out.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, want), f"replay {r}"
        plx.parallax_decode_no_alloc(other.q, other.rho, other.k, other.v, o2, scale=other.scale)
        torch.cuda.synchronize()
