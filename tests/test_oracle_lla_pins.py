"""Pins for the oracle's local linear attention (LLA) solved probe.

The pages (page "Parallax: Parameterized Local Linear Attention Gives
Transformers a 'Second Eye'", sections 1.2-1.3 and the taxonomy of 2.1): LLA
fits v ~ b + W (k - q) around each query with the softmax weights, solves a
regularised system S x = mu per token, and equals Parallax with the solved
probe rho* = S^{-1} mu; a large regulariser turns it back into softmax.

Fixed here by routes independent of the oracle's solve: the intercept of the
ridge-regularised weighted least-squares fit found by numpy.linalg.lstsq on an
augmented system; the large-lambda limit (plain softmax via scipy); the
normal equations with S_KK from numpy.cov; paged and windowed addressing
against plain slicing.  test_lla_mutants_are_caught checks that plausible
misreadings fail a pin.
"""
import numpy as np
import pytest
import scipy.special

import oracle


def rel_err(a, b):
    return float(np.max(np.abs(a - b) / (1.0 + np.abs(b))))


def ridge_intercept(q, K, V, scale, lam):
    """b of min_{b,W} sum_j p_j |v_j - b - W (k_j - q)|^2 + lam |W|_F^2 by
    numpy.linalg.lstsq: sqrt(p)-weighted data rows plus sqrt(lam) rows that
    penalise W only."""
    L, dk = K.shape
    p = scipy.special.softmax(scale * (K @ q))
    w = np.sqrt(p)[:, None]
    X = np.hstack([np.ones((L, 1)), K - q]) * w
    Y = V * w
    Xr = np.hstack([np.zeros((dk, 1)), np.sqrt(lam) * np.eye(dk)])
    coef, *_ = np.linalg.lstsq(np.vstack([X, Xr]), np.vstack([Y, np.zeros((dk, V.shape[1]))]),
                               rcond=None)
    return coef[0]


def case(seed, B=2, Hq=4, Hkv=2, L=40, dk=6, dv=5):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((B, Hq, dk)), rng.standard_normal((B, Hkv, L, dk)),
            rng.standard_normal((B, Hkv, L, dv)))


def oracle_impl(q, k, v, scale, lam, **kw):
    return oracle.lla_decode(q, k, v, scale, lam, **kw)[0]


# ------------------------------------------------------------------ pins ---
# Each takes an implementation impl(q, k, v, scale, lam, **kw) -> out.

def pin_ridge_intercept(impl):
    worst = 0.0
    for seed, lam, L in [(1, 0.3, 40), (2, 2.0, 40), (3, 0.05, 9), (4, 1e-6, 60)]:
        q, k, v = case(seed, L=L)
        out = impl(q, k, v, 0.45, lam)
        G = q.shape[1] // k.shape[1]
        for b in range(q.shape[0]):
            for h in range(q.shape[1]):
                want = ridge_intercept(q[b, h], k[b, h // G], v[b, h // G], 0.45, lam)
                worst = max(worst, rel_err(out[b, h], want))
    return worst


def pin_large_lambda_is_softmax(impl):
    """A regulariser that dominates S_KK sends rho* to 0: plain softmax."""
    q, k, v = case(5)
    out = impl(q, k, v, 0.45, 1e12)
    G = q.shape[1] // k.shape[1]
    worst = 0.0
    for b in range(q.shape[0]):
        for h in range(q.shape[1]):
            want = scipy.special.softmax(0.45 * (k[b, h // G] @ q[b, h])) @ v[b, h // G]
            worst = max(worst, rel_err(out[b, h], want))
    return worst


def pin_window_and_lengths(impl):
    """Ragged lengths and a local window equal the same rows on sliced keys."""
    q, k, v = case(6, L=50)
    lens = np.array([50, 13], dtype=np.int32)
    W = 8
    out = impl(q, k, v, 0.45, 0.4, seq_lens=lens, window=W)
    G = q.shape[1] // k.shape[1]
    worst = 0.0
    for b in range(2):
        lo = max(0, lens[b] - W)
        for h in range(q.shape[1]):
            want = ridge_intercept(q[b, h], k[b, h // G, lo:lens[b]], v[b, h // G, lo:lens[b]],
                                   0.45, 0.4)
            worst = max(worst, rel_err(out[b, h], want))
    return worst


PINS = [pin_ridge_intercept, pin_large_lambda_is_softmax, pin_window_and_lengths]


@pytest.mark.parametrize("pin", PINS, ids=lambda f: f.__name__)
def test_lla_pin(pin):
    assert pin(oracle_impl) < 1e-9


def test_normal_equations_with_numpy_cov():
    """(S_KK + lam I) rho* = kbar - q, S_KK = numpy.cov(aweights=p, bias=True)."""
    q, k, v = case(7)
    lam = 0.7
    rho = oracle.solved_probe(q, k, 0.45, lam)
    G = q.shape[1] // k.shape[1]
    for b in range(q.shape[0]):
        for h in range(q.shape[1]):
            K = k[b, h // G]
            p = scipy.special.softmax(0.45 * (K @ q[b, h]))
            S = np.cov(K.T, aweights=p, bias=True)
            assert rel_err((S + lam * np.eye(K.shape[1])) @ rho[b, h], p @ K - q[b, h]) < 1e-12


def test_paged_equals_contiguous():
    rng = np.random.default_rng(8)
    B, Hq, Hkv, P, dk = 3, 4, 2, 4, 6
    lens = np.array([10, 1, 7], dtype=np.int32)
    nblk = (lens + P - 1) // P
    NB = int(nblk.sum())
    perm = rng.permutation(NB).astype(np.int32)
    table = np.zeros((B, int(nblk.max())), dtype=np.int32)
    off = 0
    for b in range(B):
        table[b, :nblk[b]] = perm[off:off + nblk[b]]
        off += nblk[b]
    kp = rng.standard_normal((NB, Hkv, P, dk))
    vp = rng.standard_normal((NB, Hkv, P, dk))
    q = rng.standard_normal((B, Hq, dk))
    kc = np.zeros((B, Hkv, 12, dk))
    vc = np.zeros((B, Hkv, 12, dk))
    for b in range(B):
        for j in range(lens[b]):
            kc[b, :, j] = kp[table[b, j // P], :, j % P]
            vc[b, :, j] = vp[table[b, j // P], :, j % P]
    for W in (0, 3):
        op, rp = oracle.lla_decode(q, kp, vp, 0.5, 0.3, seq_lens=lens, block_table=table,
                                   window=W)
        oc, rc = oracle.lla_decode(q, kc, vc, 0.5, 0.3, seq_lens=lens, window=W)
        assert rel_err(rp, rc) < 1e-13 and rel_err(op, oc) < 1e-13


def test_empty_row_gives_zero():
    q, k, v = case(9)
    out, rho = oracle.lla_decode(q, k, v, 0.45, 0.3, seq_lens=np.array([0, 40], dtype=np.int32))
    assert np.all(rho[0] == 0) and np.all(out[0] == 0)


# ----------------------------------------------------------------- mutants ---

def _mutant(kind):
    def impl(q, k, v, scale, lam, seq_lens=None, block_table=None, window=0):
        B, Hq, dk = q.shape
        G = Hq // k.shape[1]
        rho = np.zeros_like(q)
        for b in range(B):
            L = k.shape[2] if seq_lens is None else int(seq_lens[b])
            lo = max(0, L - window) if window > 0 else 0
            for h in range(Hq):
                K = k[b, h // G, lo:L]
                p = scipy.special.softmax(scale * (K @ q[b, h]))
                if kind == "unweighted":
                    p = np.full_like(p, 1.0 / len(p))
                kbar = p @ K
                Kc = K - kbar
                S = (Kc * p[:, None]).T @ Kc
                mu = q[b, h] - kbar if kind == "mu_sign" else kbar - q[b, h]
                if kind == "uncentred":
                    S = (K * p[:, None]).T @ K
                reg = 0.0 if kind == "no_lambda" else lam
                rho[b, h] = np.linalg.solve(S + reg * np.eye(dk) + 1e-9 * np.eye(dk), mu)
        return oracle.decode(q, rho, k, v, scale, seq_lens=seq_lens, window=window)
    impl.__name__ = kind
    return impl


@pytest.mark.parametrize("kind", ["mu_sign", "unweighted", "uncentred", "no_lambda"])
def test_lla_mutants_are_caught(kind):
    impl = _mutant(kind)
    assert any(not pin(impl) < 1e-6 for pin in PINS), f"{kind} passes every pin"


def test_numpy_restatement_passes():
    """The mutants' shared code without a mistake passes every pin."""
    impl = _mutant("none")
    for pin in PINS:
        assert pin(impl) < 1e-6, pin.__name__
