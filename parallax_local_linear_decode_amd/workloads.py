"""Seeded synthetic inputs for Parallax attention.

This module only draws random tensors and lays them out; it contains none of
the attention arithmetic.  Both the HIP path's tests and the CPU oracle are
fed from here, so each side sees bit-identical inputs.

Draw order (fixed, per generator):
  decode : q, k, v, rho
  paged  : seq_lens, page permutation (CPU generator), then q, k, v, rho
  prefill: q, k, v, rho
Distributions: q, k, v ~ N(0, 1); rho ~ N(0, rho_std^2) (rho_std = 0.1).
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import torch

PAGE_SIZE = 16


def _gen(device, seed):
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def _randn(shape, g, device, dtype, std=1.0, chunk_dim0=True):
    """N(0, std^2) of `dtype`, drawn along dim 0 in slices to bound the fp32 temporaries."""
    out = torch.empty(shape, dtype=dtype, device=device)
    if len(shape) == 0 or shape[0] == 0:
        return out
    per = math.prod(shape[1:]) if len(shape) > 1 else 1
    step = max(1, (1 << 26) // max(per, 1)) if chunk_dim0 else shape[0]
    for s in range(0, shape[0], step):
        e = min(shape[0], s + step)
        t = torch.randn((e - s,) + tuple(shape[1:]), generator=g, device=device,
                        dtype=torch.float32)
        if std != 1.0:
            t.mul_(std)
        out[s:e].copy_(t)
    return out


@dataclass
class DecodeInputs:
    q: torch.Tensor          # [B, Hq, d] fp32
    rho: torch.Tensor        # [B, Hq, d] fp32
    k: torch.Tensor          # contiguous [B, Hkv, L, d] or paged [NB, Hkv, P, d]
    v: torch.Tensor
    scale: float
    seq_lens: torch.Tensor | None = None     # [B] int32
    block_table: torch.Tensor | None = None  # [B, max_blocks] int32


def decode_inputs(B, Hq, Hkv, d, L, *, kv_dtype=torch.bfloat16, seed=0, rho_std=0.1,
                  device="cpu", v_mode="iid", rho_zero=False):
    """Contiguous decode inputs: KV cache [B, Hkv, L, d], q/rho fp32 [B, Hq, d].

    v_mode="correlated" draws V = K M^T + 0.1 noise (M ~ N(0, 1/d)), which
    makes the covariance term large next to the softmax output.
    """
    g = _gen(device, seed)
    q = _randn((B, Hq, d), g, device, torch.float32)
    k = _randn((B, Hkv, L, d), g, device, kv_dtype)
    if v_mode == "iid":
        v = _randn((B, Hkv, L, d), g, device, kv_dtype)
    elif v_mode == "correlated":
        M = torch.randn((d, d), generator=g, device=device, dtype=torch.float32) / math.sqrt(d)
        noise = torch.randn((B, Hkv, L, d), generator=g, device=device, dtype=torch.float32)
        v = (k.float() @ M.T + 0.1 * noise).to(kv_dtype)
    else:
        raise ValueError(v_mode)
    rho = _randn((B, Hq, d), g, device, torch.float32, std=rho_std)
    if rho_zero:
        rho.zero_()
    return DecodeInputs(q=q, rho=rho, k=k, v=v, scale=1.0 / math.sqrt(d))


def paged_inputs(B, Hq, Hkv, d, *, ctx_lo=128, ctx_hi=32768, seq_lens=None, page=PAGE_SIZE,
                 kv_dtype=torch.bfloat16, seed=0, rho_std=0.1, rho_zero_rows=0,
                 poison=True, device="cpu", max_blocks=None):
    """Paged decode inputs.

    seq_lens ~ U{ctx_lo..ctx_hi} unless given.  Sequence b owns ceil(L_b/page)
    physical pages, taken from a random permutation of all NB pages, so its
    logical block i lives in page block_table[b, i].  One extra page (id NB)
    is filled with NaN; block-table entries past a sequence's last block point
    at it.  With poison=True the slots after a sequence's last token in its
    last page are NaN too, so any read beyond seq_lens shows up in the output.
    Query rows b < rho_zero_rows get rho = 0.
    Pool layout: k, v [NB + 1, Hkv, page, d].
    """
    gc = _gen("cpu", seed)
    if seq_lens is None:
        seq_lens = torch.randint(ctx_lo, ctx_hi + 1, (B,), generator=gc, dtype=torch.int64)
    seq_lens = torch.as_tensor(seq_lens, dtype=torch.int64).cpu()
    nblk = (seq_lens + page - 1) // page
    NB = int(nblk.sum())
    if max_blocks is None:
        max_blocks = max(1, int(nblk.max()) if B > 0 else 1)
    perm = torch.randperm(NB, generator=gc, dtype=torch.int64)
    table = torch.full((B, max_blocks), NB, dtype=torch.int32)
    off = 0
    for b in range(B):
        n = int(nblk[b])
        table[b, :n] = perm[off:off + n].to(torch.int32)
        off += n
    g = _gen(device, seed + 1)
    q = _randn((B, Hq, d), g, device, torch.float32)
    k = _randn((NB + 1, Hkv, page, d), g, device, kv_dtype)
    v = _randn((NB + 1, Hkv, page, d), g, device, kv_dtype)
    rho = _randn((B, Hq, d), g, device, torch.float32, std=rho_std)
    if rho_zero_rows:
        rho[:rho_zero_rows].zero_()
    nan = float("nan")
    k[NB].fill_(nan)
    v[NB].fill_(nan)
    if poison:
        for b in range(B):
            L = int(seq_lens[b])
            if L % page:
                last = int(table[b, L // page])
                k[last, :, L % page:, :] = nan
                v[last, :, L % page:, :] = nan
    return DecodeInputs(q=q, rho=rho, k=k, v=v, scale=1.0 / math.sqrt(d),
                        seq_lens=seq_lens.to(torch.int32).to(device),
                        block_table=table.to(device))


def prefill_inputs(B, S, Hq, Hkv, d, *, dtype=torch.bfloat16, seed=0, rho_std=0.1,
                   device="cpu"):
    """Causal prefill inputs: q, rho [B, S, Hq, d]; k, v [B, S, Hkv, d]."""
    g = _gen(device, seed)
    q = _randn((B, S, Hq, d), g, device, dtype)
    k = _randn((B, S, Hkv, d), g, device, dtype)
    v = _randn((B, S, Hkv, d), g, device, dtype)
    rho = _randn((B, S, Hq, d), g, device, dtype, std=rho_std)
    return q, rho, k, v, 1.0 / math.sqrt(d)


def prefill_dout(B, S, Hq, d, *, dtype=torch.bfloat16, seed=0, std=1.0, device="cpu"):
    """Upstream gradient of a prefill output, [B, S, Hq, d] ~ N(0, std^2),
    drawn from its own generator (pass a seed different from the inputs')."""
    return _randn((B, S, Hq, d), _gen(device, seed), device, dtype, std=std)


def host_array(t: torch.Tensor):
    """A numpy view of a tensor's exact bits on the host (bf16 -> raw uint16)."""
    t = t.detach().contiguous().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view("uint16")
    return t.numpy()
