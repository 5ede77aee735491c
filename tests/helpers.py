"""Shared test helpers: parity metrics and oracle calls on torch inputs."""
import numpy as np
import torch

import oracle
from parallax_local_linear_decode_amd.workloads import host_array

# Tolerances: max |gpu - ref| <= TAU * (1 + |ref|) elementwise, plus a
# relative-RMS gate ||gpu - ref|| / ||ref|| (see the tolerance derivation in
# the design notes).
TAU_F32 = 1e-5
TAU_BF16 = 2e-2
RMS_DECODE_BF16 = 1e-3
RMS_PREFILL = 1e-2
# Prefill backward: the forward keeps its statistics from bf16-rounded softmax
# numerators and the backward rounds its weights p (1 + r - t), ds and dt to
# bf16; tests/test_backward_tolerance.py models both roundings in fp64 at the
# shapes of the GPU tests and checks that this bound is at least twice the
# modelled worst ratio (4.8e-2, drho: a cancelling sum) and at most four times.
TAU_BWD = 0.1
RMS_BWD = 1e-2


def parity(gpu, ref):
    """(max elementwise |g-r|/(1+|r|), relative RMS error) of gpu vs ref."""
    g = gpu.detach().double().cpu().numpy() if isinstance(gpu, torch.Tensor) else np.asarray(gpu)
    r = np.asarray(ref, dtype=np.float64)
    assert g.shape == r.shape, (g.shape, r.shape)
    assert np.all(np.isfinite(g)), "non-finite values in GPU output"
    err = np.abs(g - r)
    ratio = float(np.max(err / (1.0 + np.abs(r)))) if err.size else 0.0
    den = float(np.linalg.norm(r))
    rms = float(np.linalg.norm(g - r) / den) if den > 0 else float(np.linalg.norm(g - r))
    return ratio, rms


def assert_parity(gpu, ref, tau, rms_gate=None, what=""):
    ratio, rms = parity(gpu, ref)
    assert ratio <= tau, f"{what}: max err ratio {ratio:.3e} > {tau:.1e} (rel-RMS {rms:.3e})"
    if rms_gate is not None:
        assert rms <= rms_gate, f"{what}: rel-RMS {rms:.3e} > {rms_gate:.1e}"
    return ratio, rms


def oracle_decode(inp, *, form="streaming", seq_lens=None, rows=None, window=0):
    """Run the oracle on a DecodeInputs (torch tensors, any device)."""
    sl = inp.seq_lens if seq_lens is None else seq_lens
    sl = None if sl is None else host_array(sl).astype(np.int32)
    bt = None if inp.block_table is None else host_array(inp.block_table)
    return oracle.decode(host_array(inp.q), host_array(inp.rho), host_array(inp.k),
                         host_array(inp.v), inp.scale, seq_lens=sl, block_table=bt, form=form,
                         window=window)


def gather_sequences(inp, batch_ids):
    """The paged inputs restricted to `batch_ids`: a compact host pool holding
    only those sequences' pages, with a renumbered block table."""
    table = inp.block_table.cpu()
    lens = inp.seq_lens.cpu()
    P = inp.k.shape[2]
    pages = []
    for b in batch_ids:
        n = (int(lens[b]) + P - 1) // P
        pages.append(table[b, :n].long())
    all_ids = torch.cat(pages) if pages else torch.zeros(0, dtype=torch.long)
    kk = inp.k[all_ids.to(inp.k.device)].cpu()
    vv = inp.v[all_ids.to(inp.v.device)].cpu()
    maxb = max(1, max(len(x) for x in pages))
    new_table = np.zeros((len(batch_ids), maxb), dtype=np.int32)
    off = 0
    for i, ids in enumerate(pages):
        new_table[i, :len(ids)] = np.arange(off, off + len(ids), dtype=np.int32)
        off += len(ids)
    idx = torch.as_tensor(batch_ids, dtype=torch.long)
    return (host_array(inp.q.cpu()[idx]), host_array(inp.rho.cpu()[idx]), host_array(kk),
            host_array(vv), lens[idx].numpy().astype(np.int32), new_table)
