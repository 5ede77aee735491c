"""Pins for the fp64 oracle: each check is fixed by something other than the
oracle itself -- a hand-worked example, a closed form, a library routine
(scipy softmax, numpy.cov, numpy.linalg.lstsq), an algebraic invariant of the
definition, or brute force on tiny inputs.

The definition pinned here (page "Parallax: Parameterized Local Linear
Attention Gives Transformers a 'Second Eye'", section 1.3): o = o_SA - S_KV rho
with S_KV the softmax-weighted covariance of values against keys.
"""
import math

import numpy as np
import pytest
import scipy.special

import oracle

FORMS = ["explicit", "streaming"]


def one_row(form):
    """The oracle on a single (batch, head) row: q, rho [dk], K [L, dk], V [L, dv]."""
    def impl(q, rho, K, V, scale):
        return oracle.decode(q[None, None], rho[None, None], K[None, None], V[None, None],
                             scale, form=form, threads=1)[0, 0]
    return impl


def rand_row(rng, L, dk, dv, rho_std=0.5):
    return (rng.standard_normal(dk), rho_std * rng.standard_normal(dk),
            rng.standard_normal((L, dk)), rng.standard_normal((L, dv)))


def rel_err(a, b):
    return float(np.max(np.abs(a - b) / (1.0 + np.abs(b))))


# ------------------------------------------------------------------ pins ---
# Each pin takes an implementation of one row and returns its max relative
# deviation from the pinned value.  test_mutants_are_caught checks that every
# plausible mistake fails at least one of them.

def pin_hand_example(impl):
    """Worked by hand: scale 1, q = 1, keys (0, ln 3) -> p = (1/4, 3/4);
    values (0, 4) -> o_SA = 3; cov = p1 p2 (v1-v2)(k1-k2) = (3/16)(-4)(-ln 3)
    = (3/4) ln 3; rho = 1 -> o = 3 - (3/4) ln 3."""
    o = impl(np.array([1.0]), np.array([1.0]), np.array([[0.0], [math.log(3.0)]]),
             np.array([[0.0], [4.0]]), 1.0)
    return rel_err(o, np.array([3.0 - 0.75 * math.log(3.0)]))


def pin_two_tokens(impl):
    """Two keys: S_KV = p1 p2 (v1 - v2)(k1 - k2)^T exactly (closed form)."""
    rng = np.random.default_rng(11)
    worst = 0.0
    for dk, dv in [(3, 5), (4, 4), (6, 2)]:
        q, rho, K, V = rand_row(rng, 2, dk, dv)
        scale = 0.7
        s1, s2 = scale * K[0] @ q, scale * K[1] @ q
        p1 = 1.0 / (1.0 + math.exp(s2 - s1))
        p2 = 1.0 - p1
        want = p1 * V[0] + p2 * V[1] - p1 * p2 * (V[0] - V[1]) * ((K[0] - K[1]) @ rho)
        worst = max(worst, rel_err(impl(q, rho, K, V, scale), want))
    return worst


def pin_numpy_cov(impl):
    """o = softmax-mean of V minus numpy's weighted (biased) cross-covariance times rho."""
    rng = np.random.default_rng(12)
    worst = 0.0
    for L, dk, dv in [(5, 3, 4), (17, 8, 8), (40, 4, 6), (64, 16, 16)]:
        q, rho, K, V = rand_row(rng, L, dk, dv)
        scale = 1.0 / math.sqrt(dk)
        p = scipy.special.softmax(scale * (K @ q))
        C = np.cov(np.vstack([V.T, K.T]), aweights=p, bias=True)[:dv, dv:]
        want = p @ V - C @ rho
        worst = max(worst, rel_err(impl(q, rho, K, V, scale), want))
    return worst


def pin_uniform_limit(impl):
    """q = 0 makes every weight 1/L (the bandwidth -> infinity end of the
    taxonomy, section 2.1): o = mean(V) - cov_unweighted(V, K) rho."""
    rng = np.random.default_rng(13)
    worst = 0.0
    for L, dk, dv in [(7, 3, 5), (33, 8, 8)]:
        _, rho, K, V = rand_row(rng, L, dk, dv)
        C = np.cov(np.vstack([V.T, K.T]), bias=True)[:dv, dv:]
        want = V.mean(axis=0) - C @ rho
        worst = max(worst, rel_err(impl(np.zeros(dk), rho, K, V, 0.5), want))
    return worst


def pin_softmax_at_rho_zero(impl):
    """rho = 0 (W_R = 0) is plain softmax attention."""
    rng = np.random.default_rng(14)
    worst = 0.0
    for L, dk, dv in [(1, 4, 4), (9, 4, 3), (128, 64, 64)]:
        q, _, K, V = rand_row(rng, L, dk, dv)
        scale = 1.0 / math.sqrt(dk)
        want = scipy.special.softmax(scale * (K @ q)) @ V
        worst = max(worst, rel_err(impl(q, np.zeros(dk), K, V, scale), want))
    return worst


def pin_lla_intercept(impl):
    """Local linear attention cross-check (sections 1.2-1.3).  The softmax-
    weighted least-squares fit v ~ b + W (k - q) has intercept
    b = vbar - S_VK S_KK^{-1} (kbar - q); so with the solved probe
    rho* = S_KK^{-1} (kbar - q) the Parallax output must equal the intercept
    that numpy.linalg.lstsq finds on sqrt(p)-weighted rows."""
    rng = np.random.default_rng(15)
    worst = 0.0
    for L, dk, dv in [(30, 3, 5), (60, 6, 4)]:
        q, _, K, V = rand_row(rng, L, dk, dv)
        scale = 0.4
        p = scipy.special.softmax(scale * (K @ q))
        kbar = p @ K
        Kc = K - kbar
        S_KK = (Kc * p[:, None]).T @ Kc
        rho_star = np.linalg.solve(S_KK, kbar - q)
        X = np.hstack([np.ones((L, 1)), K - q])
        w = np.sqrt(p)[:, None]
        coef, *_ = np.linalg.lstsq(X * w, V * w, rcond=None)
        worst = max(worst, rel_err(impl(q, rho_star, K, V, scale), coef[0]))
    return worst


def pin_single_key(impl):
    """One key: every weight is 1 and the covariance vanishes, so o = v."""
    rng = np.random.default_rng(16)
    q, rho, K, V = rand_row(rng, 1, 8, 8)
    return rel_err(impl(q, rho, K, V, 0.3), V[0])


PINS = [pin_hand_example, pin_two_tokens, pin_numpy_cov, pin_uniform_limit,
        pin_softmax_at_rho_zero, pin_lla_intercept, pin_single_key]


@pytest.mark.parametrize("form", FORMS)
@pytest.mark.parametrize("pin", PINS, ids=lambda f: f.__name__)
def test_oracle_meets_pin(form, pin):
    assert pin(one_row(form)) < 1e-12


# --------------------------------------------------- mistakes are caught ---

def _parts(q, rho, K, V, scale):
    p = scipy.special.softmax(scale * (K @ q))
    return p, p @ V, p @ K


def mut_sign(q, rho, K, V, scale):
    p, vbar, kbar = _parts(q, rho, K, V, scale)
    return vbar + ((V - vbar) * p[:, None]).T @ ((K - kbar) @ rho)


def mut_dropped_mean_term(q, rho, K, V, scale):  # o = A/Z - B/Z (A R / Z^2 dropped)
    p, vbar, _ = _parts(q, rho, K, V, scale)
    return vbar - (p * (K @ rho)) @ V


def mut_transposed(q, rho, K, V, scale):  # rho contracted on the value side
    p, vbar, kbar = _parts(q, rho, K, V, scale)
    C = ((V - vbar) * p[:, None]).T @ (K - kbar)
    return vbar - C.T @ rho if C.shape[0] == C.shape[1] else vbar * np.nan


def mut_scaled_probe(q, rho, K, V, scale):  # logit scale applied to t = rho.k too
    p, vbar, kbar = _parts(q, rho, K, V, scale)
    return vbar - ((V - vbar) * p[:, None]).T @ (scale * (K - kbar) @ rho)


def mut_unweighted_cov(q, rho, K, V, scale):
    p, vbar, _ = _parts(q, rho, K, V, scale)
    C = np.cov(np.vstack([V.T, K.T]), bias=True)[:V.shape[1], V.shape[1]:]
    return vbar - C @ rho


def mut_bessel(q, rho, K, V, scale):  # reliability-weights correction 1/(1 - sum p^2)
    p, vbar, kbar = _parts(q, rho, K, V, scale)
    C = ((V - vbar) * p[:, None]).T @ (K - kbar) / (1.0 - np.sum(p * p))
    return vbar - C @ rho


def mut_uncentred(q, rho, K, V, scale):
    p, vbar, _ = _parts(q, rho, K, V, scale)
    return vbar - (V * p[:, None]).T @ (K @ rho)


def mut_unnormalised_weights(q, rho, K, V, scale):  # exp(s) used without dividing by Z
    s = scale * (K @ q)
    e = np.exp(s - s.max())
    vbar = e @ V / e.sum()
    kbar = e @ K / e.sum()
    return vbar - ((V - vbar) * e[:, None]).T @ ((K - kbar) @ rho)


MUTANTS = [mut_sign, mut_dropped_mean_term, mut_transposed, mut_scaled_probe,
           mut_unweighted_cov, mut_bessel, mut_uncentred, mut_unnormalised_weights]


@pytest.mark.parametrize("mutant", MUTANTS, ids=lambda f: f.__name__)
def test_mutants_are_caught(mutant):
    """Every plausible mistake in the definition fails at least one pin."""
    failures = []
    for pin in PINS:
        with np.errstate(all="ignore"):
            e = pin(mutant)
        if not (e < 1e-9):
            failures.append(pin.__name__)
    assert failures, f"{mutant.__name__} passes every pin"


# ------------------------------------------------- oracle self-consistency ---

@pytest.mark.parametrize("L", [1, 2, 3, 7, 16, 33])
@pytest.mark.parametrize("d", [1, 2, 4, 8])
@pytest.mark.parametrize("G", [1, 2])
def test_streaming_equals_explicit(L, d, G):
    rng = np.random.default_rng(1000 * L + 10 * d + G)
    B, Hkv = 2, 2
    q = rng.standard_normal((B, Hkv * G, d))
    rho = 0.3 * rng.standard_normal((B, Hkv * G, d))
    k = rng.standard_normal((B, Hkv, L, d))
    v = rng.standard_normal((B, Hkv, L, d))
    a = oracle.decode(q, rho, k, v, 0.6, form="explicit")
    b = oracle.decode(q, rho, k, v, 0.6, form="streaming")
    assert rel_err(b, a) < 1e-12


@pytest.mark.parametrize("form", FORMS)
def test_single_key_is_bitwise_value(form):
    rng = np.random.default_rng(3)
    q, rho, K, V = rand_row(rng, 1, 64, 64)
    o = one_row(form)(q, rho, K, V, 0.125)
    assert np.array_equal(o, V[0])


@pytest.mark.parametrize("form", FORMS)
def test_rho_zero_bitwise_in_explicit_form(form):
    """With rho = 0 the correction is an exact zero, so o is the softmax mean."""
    rng = np.random.default_rng(4)
    q, _, K, V = rand_row(rng, 50, 8, 8)
    o0 = one_row(form)(q, np.zeros(8), K, V, 0.3)
    want = one_row("explicit")(q, np.zeros(8), K, V, 0.3)
    assert rel_err(o0, want) < 1e-14


def test_empty_row_is_zero():
    rng = np.random.default_rng(5)
    q = rng.standard_normal((3, 2, 4))
    k = rng.standard_normal((3, 2, 6, 4))
    v = rng.standard_normal((3, 2, 6, 4))
    for form in FORMS:
        o = oracle.decode(q, q, k, v, 0.5, seq_lens=np.array([6, 0, 3]), form=form)
        assert np.all(o[1] == 0.0) and np.all(np.isfinite(o))


def test_large_logits_do_not_overflow():
    """Logits in the hundreds, and a max that grows at every token."""
    rng = np.random.default_rng(6)
    d, L = 4, 40
    q = rng.standard_normal(d)
    u = q / np.linalg.norm(q)
    K = np.outer(np.arange(L), u) * 3.0 + 0.01 * rng.standard_normal((L, d))
    V = rng.standard_normal((L, d))
    rho = 0.2 * rng.standard_normal(d)
    scale = 50.0
    p = scipy.special.softmax(scale * (K @ q))
    C = np.cov(np.vstack([V.T, K.T]), aweights=p, bias=True)[:d, d:]
    want = p @ V - C @ rho
    for form in FORMS:
        o = one_row(form)(q, rho, K, V, scale)
        assert np.all(np.isfinite(o)) and rel_err(o, want) < 1e-10


def test_invariants():
    """Algebra of the definition: value shift, key shift, rho-linearity, token order."""
    rng = np.random.default_rng(7)
    L, d = 25, 6
    q, rho, K, V = rand_row(rng, L, d, d)
    f = one_row("streaming")
    s = 0.4
    c = rng.standard_normal(d)
    assert rel_err(f(q, rho, K, V + c, s), f(q, rho, K, V, s) + c) < 1e-12
    assert rel_err(f(q, rho, K + 0.5 * c, V, s), f(q, rho, K, V, s)) < 1e-12
    r2 = 0.3 * rng.standard_normal(d)
    lhs = f(q, rho + r2, K, V, s) + f(q, np.zeros(d), K, V, s)
    rhs = f(q, rho, K, V, s) + f(q, r2, K, V, s)
    assert rel_err(lhs, rhs) < 1e-12
    perm = rng.permutation(L)
    assert rel_err(f(q, rho, K[perm], V[perm], s), f(q, rho, K, V, s)) < 1e-12


def test_gqa_mapping_consecutive_groups():
    """Query head h reads KV head h // (Hq / Hkv)."""
    rng = np.random.default_rng(8)
    B, Hq, Hkv, L, d = 2, 6, 2, 9, 4
    q = rng.standard_normal((B, Hq, d))
    rho = 0.3 * rng.standard_normal((B, Hq, d))
    k = rng.standard_normal((B, Hkv, L, d))
    v = rng.standard_normal((B, Hkv, L, d))
    o = oracle.decode(q, rho, k, v, 0.5)
    G = Hq // Hkv
    for b in range(B):
        for h in range(Hq):
            ref = one_row("explicit")(q[b, h], rho[b, h], k[b, h // G], v[b, h // G], 0.5)
            assert rel_err(o[b, h], ref) < 1e-12


def test_paged_equals_contiguous_gather():
    """A shuffled page pool read through the block table equals the contiguous
    cache assembled from it with numpy indexing; slots past seq_lens are NaN."""
    rng = np.random.default_rng(9)
    B, Hq, Hkv, d, P = 4, 4, 2, 8, 16
    lens = np.array([1, 16, 17, 45], dtype=np.int32)
    nblk = (lens + P - 1) // P
    NB = int(nblk.sum())
    perm = rng.permutation(NB)
    maxb = int(nblk.max())
    table = np.full((B, maxb), NB, dtype=np.int32)
    off = 0
    for b in range(B):
        table[b, :nblk[b]] = perm[off:off + nblk[b]]
        off += nblk[b]
    kp = rng.standard_normal((NB + 1, Hkv, P, d))
    vp = rng.standard_normal((NB + 1, Hkv, P, d))
    kp[NB] = np.nan
    vp[NB] = np.nan
    for b in range(B):
        if lens[b] % P:
            kp[table[b, lens[b] // P], :, lens[b] % P:] = np.nan
            vp[table[b, lens[b] // P], :, lens[b] % P:] = np.nan
    q = rng.standard_normal((B, Hq, d))
    rho = 0.3 * rng.standard_normal((B, Hq, d))
    Lcap = maxb * P
    kc = np.zeros((B, Hkv, Lcap, d))
    vc = np.zeros((B, Hkv, Lcap, d))
    for b in range(B):
        j = np.arange(lens[b])
        kc[b, :, :lens[b]] = kp[table[b, j // P], :, j % P].transpose(1, 0, 2)
        vc[b, :, :lens[b]] = vp[table[b, j // P], :, j % P].transpose(1, 0, 2)
    for form in FORMS:
        op = oracle.decode(q, rho, kp, vp, 0.35, seq_lens=lens, block_table=table, form=form)
        oc = oracle.decode(q, rho, kc, vc, 0.35, seq_lens=lens, form=form)
        assert np.all(np.isfinite(op))
        assert np.array_equal(op, oc)


def test_bf16_widening_is_exact():
    rng = np.random.default_rng(10)
    bits = (rng.integers(0, 1 << 16, size=(1, 2, 12, 8), dtype=np.uint32) & 0xBFFF).astype(np.uint16)
    bits_v = (rng.integers(0, 1 << 16, size=(1, 2, 12, 8), dtype=np.uint32) & 0xBFFF).astype(np.uint16)
    as_f32 = lambda b: (b.astype(np.uint32) << 16).view(np.float32)
    q = rng.standard_normal((1, 4, 8)).astype(np.float32)
    rho = (0.1 * rng.standard_normal((1, 4, 8))).astype(np.float32)
    a = oracle.decode(q, rho, bits, bits_v, 0.35)
    b = oracle.decode(q, rho, as_f32(bits), as_f32(bits_v), 0.35)
    assert np.array_equal(a, b)


# ---------------------------------------------------------------- prefill ---

def _prefill_case(seed, B=2, S=37, Hq=4, Hkv=2, d=8):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, S, Hq, d))
    rho = 0.3 * rng.standard_normal((B, S, Hq, d))
    k = rng.standard_normal((B, S, Hkv, d))
    v = rng.standard_normal((B, S, Hkv, d))
    return q, rho, k, v


def test_prefill_row_is_decode_over_prefix():
    q, rho, k, v = _prefill_case(20)
    B, S, Hq, d = q.shape
    G = Hq // k.shape[2]
    rows = np.array([0, 1, 5, 17, 36], dtype=np.int32)
    for form in FORMS:
        o = oracle.prefill(q, rho, k, v, 0.4, rows=rows, form=form)
        for ri, i in enumerate(rows):
            for b in range(B):
                for h in range(Hq):
                    ref = one_row("explicit")(q[b, i, h], rho[b, i, h], k[b, :i + 1, h // G],
                                              v[b, :i + 1, h // G], 0.4)
                    assert rel_err(o[b, ri, h], ref) < 1e-12


def test_prefill_first_row_is_first_value():
    q, rho, k, v = _prefill_case(21)
    G = q.shape[2] // k.shape[2]
    o = oracle.prefill(q, rho, k, v, 0.4, rows=[0])
    for h in range(q.shape[2]):
        assert np.array_equal(o[:, 0, h], v[:, 0, h // G])


def test_prefill_rho_zero_is_causal_softmax():
    q, _, k, v = _prefill_case(22)
    B, S, Hq, d = q.shape
    G = Hq // k.shape[2]
    o = oracle.prefill(q, np.zeros_like(q), k, v, 0.4)
    mask = np.tril(np.ones((S, S), dtype=bool))
    for b in range(B):
        for h in range(Hq):
            logits = 0.4 * q[b, :, h] @ k[b, :, h // G].T
            p = scipy.special.softmax(np.where(mask, logits, -np.inf), axis=1)
            assert rel_err(o[b, :, h], p @ v[b, :, h // G]) < 1e-12


def test_prefill_uniform_limit():
    q, rho, k, v = _prefill_case(23)
    G = q.shape[2] // k.shape[2]
    o = oracle.prefill(np.zeros_like(q), rho, k, v, 0.4, rows=[3, 20, 36])
    for ri, i in enumerate([3, 20, 36]):
        for h in range(q.shape[2]):
            K, V = k[0, :i + 1, h // G], v[0, :i + 1, h // G]
            C = np.cov(np.vstack([V.T, K.T]), bias=True)[:8, 8:]
            assert rel_err(o[0, ri, h], V.mean(0) - C @ rho[0, i, h]) < 1e-12


# ---------------------------------------------------------------- window ---
# Local window W (the "local window" the Parallax page leaves open, section
# 3.1): a row keeps only its W most recent keys -- decode over L cached
# tokens uses keys L-W .. L-1, prefill row i uses keys i-W+1 .. i.

def _np_parallax(q, rho, K, V, scale):
    """The definition in numpy/scipy: softmax weights, numpy's weighted
    (biased) cross-covariance."""
    dv = V.shape[1]
    p = scipy.special.softmax(scale * (K @ q))
    if K.shape[0] == 1:
        return V[0].copy()
    C = np.cov(np.vstack([V.T, K.T]), aweights=p, bias=True)[:dv, dv:]
    return p @ V - C @ rho


def _two_token(q, rho, K, V, scale):
    """Closed form for two keys: S_KV = p1 p2 (v1 - v2)(k1 - k2)^T."""
    s1, s2 = scale * K[0] @ q, scale * K[1] @ q
    p1 = 1.0 / (1.0 + math.exp(s2 - s1))
    p2 = 1.0 - p1
    return p1 * V[0] + p2 * V[1] - p1 * p2 * (V[0] - V[1]) * ((K[0] - K[1]) @ rho)


def _window_decode_case(seed, lens=(5, 37, 64, 1), Hq=4, Hkv=2, d=6):
    rng = np.random.default_rng(seed)
    B, Lcap = len(lens), max(lens)
    q = rng.standard_normal((B, Hq, d))
    rho = 0.4 * rng.standard_normal((B, Hq, d))
    k = rng.standard_normal((B, Hkv, Lcap, d))
    v = rng.standard_normal((B, Hkv, Lcap, d))
    return q, rho, k, v, np.array(lens, dtype=np.int32)


@pytest.mark.parametrize("form", FORMS)
@pytest.mark.parametrize("W", [1, 2, 3, 16, 37, 100])
def test_window_decode_against_numpy(form, W):
    q, rho, k, v, lens = _window_decode_case(30)
    B, Hq, d = q.shape
    G = Hq // k.shape[1]
    o = oracle.decode(q, rho, k, v, 0.45, seq_lens=lens, window=W, form=form)
    for b in range(B):
        L = int(lens[b])
        j0 = max(0, L - W)
        for h in range(Hq):
            K, V = k[b, h // G, j0:L], v[b, h // G, j0:L]
            if K.shape[0] == 1:
                want = V[0]                   # one key: o = v
            elif K.shape[0] == 2:
                want = _two_token(q[b, h], rho[b, h], K, V, 0.45)
            else:
                want = _np_parallax(q[b, h], rho[b, h], K, V, 0.45)
            assert rel_err(o[b, h], want) < 1e-12, (b, h, W)


@pytest.mark.parametrize("form", FORMS)
def test_window_at_least_the_row_is_full_attention(form):
    q, rho, k, v, lens = _window_decode_case(31)
    full = oracle.decode(q, rho, k, v, 0.45, seq_lens=lens, form=form)
    for W in (64, 65, 1000):
        assert np.array_equal(oracle.decode(q, rho, k, v, 0.45, seq_lens=lens, window=W,
                                            form=form), full)


def test_window_paged_equals_contiguous_gather():
    """Windowed paged decode against numpy indexing of the same pages."""
    rng = np.random.default_rng(32)
    B, Hq, Hkv, d, P = 3, 4, 2, 6, 4
    lens = np.array([9, 14, 3], dtype=np.int32)
    nblk = (lens + P - 1) // P
    NB = int(nblk.sum())
    perm = rng.permutation(NB).astype(np.int32)
    table = np.zeros((B, int(nblk.max())), dtype=np.int32)
    off = 0
    for b in range(B):
        table[b, :nblk[b]] = perm[off:off + nblk[b]]
        off += nblk[b]
    k = rng.standard_normal((NB, Hkv, P, d))
    v = rng.standard_normal((NB, Hkv, P, d))
    q = rng.standard_normal((B, Hq, d))
    rho = 0.4 * rng.standard_normal((B, Hq, d))
    G = Hq // Hkv
    for W in (1, 5, 10):
        o = oracle.decode(q, rho, k, v, 0.5, seq_lens=lens, block_table=table, window=W)
        for b in range(B):
            L = int(lens[b])
            j = np.arange(max(0, L - W), L)
            for h in range(Hq):
                K = k[table[b, j // P], h // G, j % P]
                V = v[table[b, j // P], h // G, j % P]
                assert rel_err(o[b, h], _np_parallax(q[b, h], rho[b, h], K, V, 0.5)) < 1e-12


@pytest.mark.parametrize("form", FORMS)
@pytest.mark.parametrize("W", [1, 2, 5, 36])
def test_window_prefill_against_numpy(form, W):
    q, rho, k, v = _prefill_case(33)
    B, S, Hq, d = q.shape
    G = Hq // k.shape[2]
    rows = np.array([0, 1, 4, 5, 17, 36], dtype=np.int32)
    o = oracle.prefill(q, rho, k, v, 0.4, rows=rows, form=form, window=W)
    for ri, i in enumerate(rows):
        j0 = max(0, int(i) - W + 1)
        for b in range(B):
            for h in range(Hq):
                K, V = k[b, j0:i + 1, h // G], v[b, j0:i + 1, h // G]
                assert rel_err(o[b, ri, h], _np_parallax(q[b, i, h], rho[b, i, h], K, V, 0.4)) \
                    < 1e-12, (i, b, h, W)


def test_window_mutants_are_caught():
    """A window one key too wide, or counted from the oldest key, fails the
    numpy pin."""
    q, rho, k, v, lens = _window_decode_case(34)
    G = q.shape[1] // k.shape[1]
    W = 3
    wrong = {
        "one key too many": lambda L: (max(0, L - W - 1), L),
        "oldest keys": lambda L: (0, min(L, W)),
    }
    for name, rng_of in wrong.items():
        worst = 0.0
        for b in range(q.shape[0]):
            L = int(lens[b])
            j0, j1 = rng_of(L)
            for h in range(q.shape[1]):
                got = oracle.decode(q[b:b + 1, h:h + 1], rho[b:b + 1, h:h + 1],
                                    k[b:b + 1, h // G:h // G + 1, j0:j1],
                                    v[b:b + 1, h // G:h // G + 1, j0:j1], 0.45)[0, 0]
                lo = max(0, L - W)
                want = _np_parallax(q[b, h], rho[b, h], k[b, h // G, lo:L], v[b, h // G, lo:L],
                                    0.45)
                worst = max(worst, rel_err(got, want))
        assert worst > 1e-6, name


# ------------------------------------------------------ probe projection ---
# rho = W_R x beside q = W_Q x (section 1.3); W_R = 0 gives rho = 0, which
# the page notes turns Parallax back into plain softmax attention.

def test_qr_projection_hand_example():
    x = np.array([[1.0, 2.0], [0.5, -1.0]])
    w_q = np.array([[1.0, 0.0], [0.0, 1.0], [2.0, 3.0]])
    w_r = np.array([[1.0, 1.0], [-1.0, 0.0], [0.0, 0.0]])
    q, rho = oracle.qr_projection(x, w_q, w_r)
    assert np.array_equal(q, [[1.0, 2.0, 8.0], [0.5, -1.0, -2.0]])
    assert np.array_equal(rho, [[3.0, -1.0, 0.0], [-0.5, -0.5, 0.0]])


def test_qr_projection_brute_force_and_zero_probe():
    rng = np.random.default_rng(60)
    x, w_q, w_r = (rng.standard_normal(s) for s in ((5, 7), (4, 7), (4, 7)))
    q, rho = oracle.qr_projection(x, w_q, w_r)
    for t in range(5):
        for n in range(4):
            assert abs(q[t, n] - sum(w_q[n, k] * x[t, k] for k in range(7))) < 1e-12
            assert abs(rho[t, n] - sum(w_r[n, k] * x[t, k] for k in range(7))) < 1e-12
    assert np.all(oracle.qr_projection(x, w_q, np.zeros_like(w_r))[1] == 0)


def test_qr_projection_reads_bf16_bits_exactly():
    vals = np.array([1.0, -2.5, 0.15625, 3.0e-3], dtype=np.float32)
    bits = (vals.view(np.uint32) >> 16).astype(np.uint16)  # exactly representable in bf16
    widened = (bits.astype(np.uint32) << 16).view(np.float32)
    q, _ = oracle.qr_projection(bits[None, :], bits[None, :], bits[None, :])
    assert q[0, 0] == float(np.dot(widened.astype(np.float64), widened.astype(np.float64)))
