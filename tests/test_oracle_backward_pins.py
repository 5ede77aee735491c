"""Pins for the training side of the fp64 oracle: the forward statistics a
prefill pass keeps (log-sum-exp, r, o_SA) and the gradients of
sum(dout * out) with respect to q, rho, k, v.

The gradients are fixed by routes that share nothing with the oracle's
chain-rule code: central finite differences of the (already pinned) forward
oracle; the closed form drho = -S_KV^T dout, which holds because out is linear
in rho (page "Parallax: Parameterized Local Linear Attention Gives
Transformers a 'Second Eye'", section 1.3: out = o_SA - S_KV rho), with S_KV
from numpy.cov; torch autograd through scaled_dot_product_attention at
rho = 0 (plain softmax attention); torch autograd through the covariance
definition written with torch ops; and two invariants (values enter out only
through o_SA once the covariance is centred, so the value gradients of a KV
head sum to the summed dout of its rows; a common shift of all keys changes
nothing, so the key gradients sum to zero).  test_backward_mutants_are_caught
checks that each plausible mistake in the chain rule fails one of them.
"""
import numpy as np
import pytest
import scipy.special
import torch

import oracle


CASES = {
    # name: (B, S, Hq, Hkv, d, window, seed)
    "mha": (1, 6, 2, 2, 4, 0, 1),
    "gqa": (2, 7, 4, 2, 5, 0, 2),
    "gqa_window": (1, 9, 4, 2, 3, 3, 3),
    "window1": (1, 5, 2, 1, 4, 1, 4),
}


def make_case(name, rho_zero=False):
    B, S, Hq, Hkv, d, W, seed = CASES[name]
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, S, Hq, d))
    rho = np.zeros((B, S, Hq, d)) if rho_zero else 0.5 * rng.standard_normal((B, S, Hq, d))
    k = rng.standard_normal((B, S, Hkv, d))
    v = rng.standard_normal((B, S, Hkv, d))
    g = rng.standard_normal((B, S, Hq, d))
    return q, rho, k, v, g, 0.6, W


def oracle_impl(q, rho, k, v, g, scale, W):
    return oracle.prefill_backward(q, rho, k, v, g, scale, window=W, threads=1)


def rel_err(a, b):
    return float(np.max(np.abs(a - b)) / (1.0 + np.max(np.abs(b))))


def worst(grads, ref):
    return max(rel_err(x, y) for x, y in zip(grads, ref))


# ------------------------------------------------------------- references ---

_FD_CACHE = {}


def finite_differences(name):
    """Central differences (h = 1e-6) of sum(g * out) with out from the
    forward oracle's explicit form, for every element of q, rho, k, v."""
    if name in _FD_CACHE:
        return _FD_CACHE[name]
    q, rho, k, v, g, scale, W = make_case(name)
    args = {"q": q, "rho": rho, "k": k, "v": v}

    def loss(a):
        out = oracle.prefill(a["q"], a["rho"], a["k"], a["v"], scale, form="explicit",
                             window=W, threads=1)
        return float(np.sum(g * out))

    h = 1e-6
    res = []
    for key in ("q", "rho", "k", "v"):
        X = args[key]
        num = np.zeros_like(X)
        for idx in np.ndindex(X.shape):
            a = dict(args)
            Xp = X.copy()
            Xp[idx] += h
            a[key] = Xp
            lp = loss(a)
            Xm = X.copy()
            Xm[idx] -= h
            a[key] = Xm
            num[idx] = (lp - loss(a)) / (2 * h)
        res.append(num)
    _FD_CACHE[name] = res
    return res


def torch_definition(q, rho, k, v, g, scale, W):
    """Autograd through the definition written with torch ops: causal (and
    windowed) softmax weights, weighted means, the explicit covariance
    matrix, out = o_SA - S_KV rho."""
    B, S, Hq, d = q.shape
    G = Hq // k.shape[2]
    tq, tr, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, rho, k, v))
    kk = tk.repeat_interleave(G, dim=2)
    vv = tv.repeat_interleave(G, dim=2)
    i = torch.arange(S)[:, None]
    j = torch.arange(S)[None, :]
    keep = j <= i
    if W > 0:
        keep = keep & (j > i - W)
    s = scale * torch.einsum("bihe,bjhe->bhij", tq, kk)
    s = s.masked_fill(~keep, float("-inf"))
    p = torch.softmax(s, dim=-1)                                  # [B, H, i, j]
    vbar = torch.einsum("bhij,bjhc->bihc", p, vv)
    kbar = torch.einsum("bhij,bjhe->bihe", p, kk)
    vc = vv[:, None, :, :, :] - vbar[:, :, None, :, :]           # [B, i, j, H, d]
    kc = kk[:, None, :, :, :] - kbar[:, :, None, :, :]
    cov = torch.einsum("bhij,bijhc,bijhe->bihce", p, vc, kc)     # [B, i, H, dv, dk]
    out = vbar - torch.einsum("bihce,bihe->bihc", cov, tr)
    (out * torch.tensor(g)).sum().backward()
    return [t.grad.numpy() for t in (tq, tr, tk, tv)]


# ------------------------------------------------------------------ pins ---
# Each pin takes an implementation of the backward and a case name and
# returns its worst relative deviation from the pinned values.

def pin_finite_differences(impl, name):
    return worst(impl(*make_case(name)), finite_differences(name))


def pin_rho_closed_form(impl, name):
    """drho_i = -S_KV(i)^T g_i, S_KV from numpy.cov with the softmax weights."""
    q, rho, k, v, g, scale, W = make_case(name)
    B, S, Hq, d = q.shape
    G = Hq // k.shape[2]
    drho = impl(q, rho, k, v, g, scale, W)[1]
    want = np.zeros_like(drho)
    for b in range(B):
        for h in range(Hq):
            for i in range(S):
                j0 = max(0, i - W + 1) if W > 0 else 0
                K, V = k[b, j0:i + 1, h // G], v[b, j0:i + 1, h // G]
                p = scipy.special.softmax(scale * (K @ q[b, i, h]))
                if K.shape[0] == 1:
                    cov = np.zeros((d, d))
                else:
                    cov = np.cov(np.hstack([V, K]).T, aweights=p, bias=True)[:d, d:]
                want[b, i, h] = -cov.T @ g[b, i, h]
    return rel_err(drho, want)


def pin_sdpa_at_rho_zero(impl, name):
    """rho = 0 is plain softmax attention: torch's scaled_dot_product_attention
    (fp64, CPU) with autograd gives dq, dk, dv."""
    q, rho, k, v, g, scale, W = make_case(name, rho_zero=True)
    B, S, Hq, d = q.shape
    G = Hq // k.shape[2]
    tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    i = torch.arange(S)[:, None]
    j = torch.arange(S)[None, :]
    keep = j <= i
    if W > 0:
        keep = keep & (j > i - W)
    out = torch.nn.functional.scaled_dot_product_attention(
        tq.transpose(1, 2), tk.repeat_interleave(G, dim=2).transpose(1, 2),
        tv.repeat_interleave(G, dim=2).transpose(1, 2), attn_mask=keep, scale=scale)
    (out.transpose(1, 2) * torch.tensor(g)).sum().backward()
    got = impl(q, rho, k, v, g, scale, W)
    return worst([got[0], got[2], got[3]], [tq.grad.numpy(), tk.grad.numpy(), tv.grad.numpy()])


def pin_autograd_definition(impl, name):
    q, rho, k, v, g, scale, W = make_case(name)
    return worst(impl(q, rho, k, v, g, scale, W), torch_definition(q, rho, k, v, g, scale, W))


def pin_invariants(impl, name):
    """Per (batch, KV head): sum_j dv_j = sum of g over the rows of its query
    heads; sum_j dk_j = 0."""
    q, rho, k, v, g, scale, W = make_case(name)
    B, S, Hq, d = q.shape
    Hkv = k.shape[2]
    G = Hq // Hkv
    _, _, dk, dv = impl(q, rho, k, v, g, scale, W)
    want_v = g.reshape(B, S, Hkv, G, d).sum(axis=(1, 3))
    return max(rel_err(dv.sum(axis=1), want_v), rel_err(dk.sum(axis=1), np.zeros_like(want_v)))


PINS = [pin_finite_differences, pin_rho_closed_form, pin_sdpa_at_rho_zero,
        pin_autograd_definition, pin_invariants]


@pytest.mark.parametrize("name", list(CASES))
@pytest.mark.parametrize("pin", PINS, ids=lambda f: f.__name__)
def test_backward_pin(pin, name):
    tol = 1e-7 if pin is pin_finite_differences else 1e-11
    assert pin(oracle_impl, name) < tol


# ----------------------------------------------------------------- mutants ---
# A numpy restatement of the chain rule with one planted mistake each.

def numpy_backward(q, rho, k, v, g, scale, W, mistake=None):
    B, S, Hq, d = q.shape
    Hkv = k.shape[2]
    G = Hq // Hkv
    dq = np.zeros_like(q)
    drho = np.zeros_like(rho)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for b in range(B):
        for h in range(Hq):
            hk = h // G
            for i in range(S):
                wl = W + 1 if mistake == "window_one_wider" else W
                j0 = max(0, i - wl + 1) if wl > 0 else 0
                K, V = k[b, j0:i + 1, hk], v[b, j0:i + 1, hk]
                p = scipy.special.softmax(scale * (K @ q[b, i, h]))
                t = K @ rho[b, i, h]
                a = p @ V
                r = p @ t
                gi = g[b, i, h]
                gA = gi if mistake == "no_one_plus_r" else (1 + r) * gi
                gB = gi if mistake == "gB_sign" else -gi
                gR = a @ gi
                dp = V @ gA + gR * t + t * (V @ gB)
                dt = p * (gR + V @ gB)
                dvj = p[:, None] * (gA[None, :] + (0 if mistake == "dv_no_t_term" else
                                                   t[:, None] * gB[None, :]))
                ds = p * dp if mistake == "softmax_no_centering" else p * (dp - p @ dp)
                dq[b, i, h] = scale * ds @ K
                drho[b, i, h] = (scale if mistake == "scaled_drho" else 1.0) * dt @ K
                dkj = scale * ds[:, None] * q[b, i, h][None, :]
                if mistake != "dk_no_probe_term":
                    dkj = dkj + dt[:, None] * rho[b, i, h][None, :]
                dk[b, j0:i + 1, hk] += dkj
                dv[b, j0:i + 1, hk] += dvj
    return dq, drho, dk, dv


MISTAKES = ["no_one_plus_r", "gB_sign", "dv_no_t_term", "softmax_no_centering", "scaled_drho",
            "dk_no_probe_term", "window_one_wider"]


def test_numpy_restatement_passes_every_pin():
    """Without a planted mistake the numpy restatement passes every pin, so a
    mutant's failure is due to its mistake."""
    for name in CASES:
        for pin in PINS:
            tol = 1e-7 if pin is pin_finite_differences else 1e-10
            assert pin(numpy_backward, name) < tol, (pin.__name__, name)


@pytest.mark.parametrize("mistake", MISTAKES)
def test_backward_mutants_are_caught(mistake):
    def impl(*a):
        return numpy_backward(*a, mistake=mistake)
    failed = [(pin.__name__, name) for pin in PINS for name in CASES
              if not pin(impl, name) < 1e-6]
    assert failed, f"{mistake} passes every pin"


# ------------------------------------------------------------------ stats ---

@pytest.mark.parametrize("name", list(CASES))
def test_stats_against_scipy(name):
    """lse against scipy.special.logsumexp; r and o_SA from scipy softmax
    weights; o_SA also equals the forward oracle's output at rho = 0."""
    q, rho, k, v, g, scale, W = make_case(name)
    B, S, Hq, d = q.shape
    G = Hq // k.shape[2]
    lse, r, a = oracle.prefill_stats(q, rho, k, v, scale, window=W, threads=1)
    for b in range(B):
        for h in range(Hq):
            for i in range(S):
                j0 = max(0, i - W + 1) if W > 0 else 0
                K, V = k[b, j0:i + 1, h // G], v[b, j0:i + 1, h // G]
                s = scale * (K @ q[b, i, h])
                p = scipy.special.softmax(s)
                assert abs(lse[b, i, h] - scipy.special.logsumexp(s)) < 1e-12
                assert abs(r[b, i, h] - p @ (K @ rho[b, i, h])) < 1e-12
                assert rel_err(a[b, i, h], p @ V) < 1e-12
    o0 = oracle.prefill(q, np.zeros_like(rho), k, v, scale, window=W)
    assert rel_err(a, o0) < 1e-12


def test_stats_rows_subset():
    q, rho, k, v, g, scale, W = make_case("gqa")
    full = oracle.prefill_stats(q, rho, k, v, scale)
    rows = np.array([6, 0, 3], dtype=np.int32)
    sub = oracle.prefill_stats(q, rho, k, v, scale, rows=rows)
    for x, y in zip(full, sub):
        assert np.array_equal(x[:, rows], y)


def test_backward_row_subset_gives_exact_late_keys():
    """With rows lo..S-1 only, dq/drho of those rows and dk/dv of keys >= lo
    equal the full gradients (no earlier row sees those keys)."""
    q, rho, k, v, g, scale, W = make_case("gqa")
    S = q.shape[1]
    full = oracle.prefill_backward(q, rho, k, v, g, scale)
    lo = 4
    rows = np.arange(lo, S, dtype=np.int32)
    dq, drho, dk, dv = oracle.prefill_backward(q, rho, k, v, g, scale, rows=rows)
    assert rel_err(dq, full[0][:, lo:]) < 1e-13
    assert rel_err(drho, full[1][:, lo:]) < 1e-13
    assert rel_err(dk[:, lo:], full[2][:, lo:]) < 1e-13
    assert rel_err(dv[:, lo:], full[3][:, lo:]) < 1e-13


def test_backward_threads_bitwise():
    q, rho, k, v, g, scale, W = make_case("gqa")
    one = oracle.prefill_backward(q, rho, k, v, g, scale, threads=1)
    many = oracle.prefill_backward(q, rho, k, v, g, scale, threads=4)
    for x, y in zip(one, many):
        assert np.array_equal(x, y)


def test_backward_rejects_bad_arguments():
    q, rho, k, v, g, scale, W = make_case("mha")
    with pytest.raises(ValueError):
        oracle.prefill_backward(q, rho, k, v, g[:, :3], scale)
    with pytest.raises(ValueError):
        oracle.prefill_backward(q, rho, k, v, g, scale, rows=np.array([99], dtype=np.int32))
    with pytest.raises(ValueError):
        oracle.prefill_backward(q, rho, k, v, g, scale, window=-1)
