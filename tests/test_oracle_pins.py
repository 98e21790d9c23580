"""Pins of the CPU oracle against facts that do not come from the oracle.

Each test names what fixes the expected value: the pages (golden fixtures,
with citations), a closed form of the Newton-Schulz iteration, a library
routine (numpy SVD / norm / unpackbits, torch's bf16 conversion), exact
rational arithmetic, or brute-force counting. The oracle's arithmetic is
never retyped here.
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import synthetic

F32, BF16, F64 = oracle.F32, oracle.BF16, oracle.F64


# ---------------------------------------------------------------------------
# independent helpers
# ---------------------------------------------------------------------------
def exact_round_f32(q: Fraction) -> np.float32:
    """Nearest fp32 to the exact rational q, ties to even (brute force over the
    three fp32 neighbours of a first guess)."""
    guess = np.float32(float(q))
    cands = [np.nextafter(guess, np.float32(-np.inf)), guess,
             np.nextafter(guess, np.float32(np.inf))]

    def key(c):
        return (abs(Fraction(float(c)) - q), int(np.array(c, np.float32).view(np.uint32)) & 1)

    return min(cands, key=key)


def torch_bf16_bits(x_f32: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(x_f32, np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def torch_round_ns(v: float, mode: int) -> float:
    if mode == F64:
        return v
    f = torch.tensor(v, dtype=torch.float64).to(torch.float32)
    if mode == BF16:
        f = f.to(torch.bfloat16).to(torch.float32)
    return float(f)


def scalar_map(s, k):
    """Newton-Schulz acts on each singular value by p(s) = 1.5 s - 0.5 s^3."""
    for _ in range(k):
        s = 1.5 * s - 0.5 * s ** 3
    return s


def rel_fro(a, b):
    return np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300)


# ---------------------------------------------------------------------------
# storage rounding
# ---------------------------------------------------------------------------
def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(1)
    x = rng.standard_normal(200_000).astype(np.float32) * np.float32(3.0)
    # exact ties between two bf16 neighbours, both parities, both signs
    base = rng.integers(0, 1 << 15, 4096).astype(np.uint32) << 16
    ties = (base | 0x8000).view(np.float32)
    extra = np.array([0.0, -0.0, np.inf, -np.inf, 3.3895313892515355e38, 1e-40, -1e-45],
                     np.float32)
    allx = np.concatenate([x, ties, -ties, extra])
    allx = allx[np.isfinite(allx) | np.isinf(allx)]
    np.testing.assert_array_equal(oracle.bf16_from_f32(allx), torch_bf16_bits(allx))
    nan = oracle.bf16_from_f32(np.array([np.nan], np.float32))
    assert np.isnan(oracle.bf16_to_f32(nan))[0]


def test_bf16_to_f32_is_exact_widening():
    h = np.arange(0, 1 << 16, dtype=np.uint32).astype(np.uint16)
    f = oracle.bf16_to_f32(h)
    ref = torch.from_numpy(h.view(np.int16).copy()).view(torch.bfloat16).to(torch.float32).numpy()
    finite = np.isfinite(ref)
    np.testing.assert_array_equal(f[finite], ref[finite])


# ---------------------------------------------------------------------------
# O1 momentum
# ---------------------------------------------------------------------------
def test_momentum_fp32_is_correctly_rounded_fma():
    rng = np.random.default_rng(2)
    n = 3000
    g = rng.standard_normal(n).astype(np.float32)
    m = rng.standard_normal(n).astype(np.float32)
    beta = np.float32(0.9)
    out = m.copy()
    oracle.momentum(g, out, float(beta))
    for i in range(n):
        q = Fraction(float(beta)) * Fraction(float(m[i])) + Fraction(float(g[i]))
        assert out[i] == exact_round_f32(q), i


def test_momentum_bf16_storage_rounds_the_fma_result():
    rng = np.random.default_rng(3)
    n = 2000
    g = rng.standard_normal(n).astype(np.float32)
    m_bits = torch_bf16_bits(rng.standard_normal(n).astype(np.float32))
    m_vals = oracle.bf16_to_f32(m_bits)
    beta = np.float32(0.9)
    out = m_bits.copy()
    oracle.momentum(g, out, float(beta))
    ref32 = np.array([exact_round_f32(Fraction(float(beta)) * Fraction(float(m_vals[i]))
                                      + Fraction(float(g[i]))) for i in range(n)], np.float32)
    np.testing.assert_array_equal(out, torch_bf16_bits(ref32))


@pytest.mark.parametrize("store", ["f32", "bf16"])
def test_momentum_special_cases(store):
    rng = np.random.default_rng(4)
    g = rng.standard_normal(1000).astype(np.float32)
    zero = np.zeros(1000, np.float32) if store == "f32" else np.zeros(1000, np.uint16)
    # first step from M0 = 0, any beta: M' = storage(G)
    first = zero.copy()
    oracle.momentum(g, first, 0.9)
    expect = g if store == "f32" else torch_bf16_bits(g)
    np.testing.assert_array_equal(first, expect)
    # beta = 0 forgets the state
    m = (rng.standard_normal(1000).astype(np.float32) if store == "f32"
         else torch_bf16_bits(rng.standard_normal(1000).astype(np.float32)))
    oracle.momentum(g, m, 0.0)
    np.testing.assert_array_equal(m, expect)
    # dyadic inputs: 0.5 * M + G exact
    md = (rng.integers(-64, 64, 1000) / 16.0).astype(np.float32)
    gd = (rng.integers(-64, 64, 1000) / 32.0).astype(np.float32)
    if store == "f32":
        mm = md.copy()
        oracle.momentum(gd, mm, 0.5)
        np.testing.assert_array_equal(mm, 0.5 * md + gd)


# ---------------------------------------------------------------------------
# O2 normalisation
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("store", ["f32", "bf16"])
def test_normalise_matches_library_norm(store):
    m = synthetic.random_matrix(5, (37, 53))
    if store == "bf16":
        m = oracle.bf16_from_f32(m)
        vals = oracle.bf16_to_f32(m).astype(np.float64)
    else:
        vals = m.astype(np.float64)
    nu, x0 = oracle.normalise(m)
    assert abs(nu - np.linalg.norm(vals)) <= 1e-14 * nu
    assert abs(np.linalg.norm(x0) - 1.0) <= 1e-14
    np.testing.assert_allclose(x0, vals / np.linalg.norm(vals), rtol=1e-14, atol=0)


def test_normalise_zero_matrix_gives_zero():
    nu, x0 = oracle.normalise(np.zeros((4, 6), np.float32))
    assert nu == 0.0 and not x0.any()


# ---------------------------------------------------------------------------
# O3 Newton-Schulz: closed forms
# ---------------------------------------------------------------------------
SHAPES = [(1, 1), (1, 5), (5, 1), (3, 3), (4, 9), (9, 4), (7, 13), (13, 7), (16, 16), (2, 16)]


@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("k", [0, 1, 2, 3, 5, 8])
def test_ns_acts_on_singular_values_by_the_cubic(shape, k):
    """With exact storage, X_k = U diag(p^k(sigma)) V^T for the SVD of X_0
    (numpy's LAPACK SVD as the independent reference)."""
    m = synthetic.random_matrix(100 + shape[0] * 31 + shape[1], shape)
    _, x0 = oracle.normalise(m)
    u = oracle.newton_schulz(x0, k, F64)
    us, s, vt = np.linalg.svd(x0, full_matrices=False)
    expect = (us * scalar_map(s, k)) @ vt
    assert rel_fro(u, expect) < 1e-12


@pytest.mark.parametrize("shape", [(6, 6), (5, 11), (11, 5), (16, 9)])
def test_ns_converges_to_polar_factor(shape):
    m = synthetic.random_matrix(7 + shape[0], shape)
    _, x0 = oracle.normalise(m)
    us, s, vt = np.linalg.svd(x0, full_matrices=False)
    assert s.min() > 1e-3  # full rank: the polar factor is unique
    prev = None
    for k in range(0, 12):
        sk = np.linalg.svd(oracle.newton_schulz(x0, k, F64), compute_uv=False)
        if prev is not None:  # singular values only grow toward 1
            assert (np.sort(sk) >= np.sort(prev) - 1e-13).all()
        prev = sk
    u = oracle.newton_schulz(x0, 80, F64)
    assert rel_fro(u, us @ vt) < 1e-10
    np.testing.assert_allclose(np.linalg.svd(u, compute_uv=False), 1.0, atol=1e-10)


@pytest.mark.parametrize("shape", [(8, 8), (6, 15), (15, 6)])
def test_ns_spectral_norm_at_most_one(shape):
    """Frobenius scaling bounds the direction's spectral norm by 1 (section 3
    'Geometry' of the summary; fr/ar/ko pages say 'at most 1') and the cubic
    keeps it there."""
    for seed in range(5):
        m = synthetic.random_matrix(50 + seed, shape, dist="student_t3")
        _, x0 = oracle.normalise(m)
        for k in range(0, 7):
            assert np.linalg.norm(oracle.newton_schulz(x0, k, F64), 2) <= 1 + 1e-12


def test_ns_rank_one_is_fixed_point():
    # small integers: the outer product is exact in fp32, so M has rank one
    rng = np.random.default_rng(11)
    a = rng.integers(-8, 9, (5, 1)).astype(np.float64)
    b = rng.integers(-8, 9, (1, 9)).astype(np.float64)
    a[0, 0], b[0, 0] = 3.0, -5.0
    _, x0 = oracle.normalise((a @ b).astype(np.float32))
    for k in (1, 3, 6):
        assert rel_fro(oracle.newton_schulz(x0, k, F64), x0) < 1e-13


def signed_partial_permutation(R, C, seed):
    rng = np.random.default_rng(seed)
    r = min(R, C)
    m = np.zeros((R, C), np.float32)
    cols = rng.permutation(max(R, C))[:r]
    signs = rng.choice([-1.0, 1.0], r).astype(np.float32)
    for t in range(r):
        if R <= C:
            m[t, cols[t]] = signs[t]
        else:
            m[cols[t], t] = signs[t]
    return m


@pytest.mark.parametrize("mode", [F32, BF16, F64])
@pytest.mark.parametrize("shape", [(4, 4), (3, 10), (10, 3), (5, 8), (8, 5)])
@pytest.mark.parametrize("k", [1, 2, 3, 5])
def test_ns_rounding_points_on_signed_permutation(mode, shape, k):
    """M = signed partial permutation: every iterate is x_j times M, where the
    scalar x_j follows the cubic with the Gram value and every iterate before
    the last stored in the working type (torch's conversions round here)."""
    m = signed_partial_permutation(*shape, seed=k + 10 * shape[0])
    _, x0 = oracle.normalise(m)
    u = oracle.newton_schulz(x0, k, mode)
    x = 1.0 / math.sqrt(min(shape))
    for j in range(k):
        a = torch_round_ns(x * x, mode)
        nxt = 1.5 * x - 0.5 * (a * x)
        x = nxt if j == k - 1 else torch_round_ns(nxt, mode)
    np.testing.assert_array_equal(u, x * m.astype(np.float64))


# ---------------------------------------------------------------------------
# O3 invariants (all storage modes)
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("mode", [F32, BF16, F64])
@pytest.mark.parametrize("shape", [(6, 17), (17, 6), (1, 9)])
def test_ns_transpose_equivariance_exact(mode, shape):
    """NS(X^T) = NS(X)^T bitwise: the tall branch on X^T sums the same
    products in the same order as the wide branch on X."""
    m = synthetic.random_matrix(21 + shape[0], shape)
    _, x0 = oracle.normalise(m)
    for k in (1, 2, 4):
        a = oracle.newton_schulz(x0, k, mode)
        b = oracle.newton_schulz(np.ascontiguousarray(x0.T), k, mode)
        np.testing.assert_array_equal(a, b.T)


@pytest.mark.parametrize("mode", [F32, BF16, F64])
def test_ns_odd_and_scale_invariance_exact(mode):
    m = synthetic.random_matrix(31, (9, 14))
    _, x0 = oracle.normalise(m)
    _, x0n = oracle.normalise(-m)
    _, x0s = oracle.normalise(m * np.float32(2.0 ** -7))
    for k in (1, 3):
        u = oracle.newton_schulz(x0, k, mode)
        np.testing.assert_array_equal(oracle.newton_schulz(x0n, k, mode), -u)
        np.testing.assert_array_equal(oracle.newton_schulz(x0s, k, mode), u)


@pytest.mark.parametrize("mode", [F32, BF16])
def test_ns_storage_modes_close_to_exact(mode):
    m = synthetic.random_matrix(41, (24, 40))
    _, x0 = oracle.normalise(m)
    tol = 1e-5 if mode == F32 else 2e-2
    for k in (1, 5):
        exact = oracle.newton_schulz(x0, k, F64)
        assert rel_fro(oracle.newton_schulz(x0, k, mode), exact) < tol


@pytest.mark.parametrize("mode", [F32, BF16, F64])
@pytest.mark.parametrize("shape", [(12, 30), (30, 12), (16, 16)])
def test_ns1_entries_equal_full_iteration(mode, shape):
    m = synthetic.random_matrix(61, shape)
    _, x0 = oracle.normalise(m)
    full = oracle.newton_schulz(x0, 1, mode)
    rng = np.random.default_rng(0)
    ri = rng.integers(0, shape[0], 50)
    ci = rng.integers(0, shape[1], 50)
    np.testing.assert_array_equal(oracle.ns1_entries(x0, mode, ri, ci), full[ri, ci])


# ---------------------------------------------------------------------------
# O4 + O5 sign and pack
# ---------------------------------------------------------------------------
def _runs_to_array(runs):
    vals = []
    for v, cnt in runs:
        x = {"nan": np.nan, "-0": -0.0}.get(v, v) if isinstance(v, str) else float(v)
        vals += [x] * cnt
    return np.array(vals, np.float32)


def test_pack_golden_vectors(golden_dir):
    spec = json.load(open(os.path.join(golden_dir, "pack_vectors.json")))
    for case in spec["cases"]:
        u = _runs_to_array(case["runs"])
        expect = np.array([int(h, 16) for h in case["expected_words_hex"]], np.uint64)
        for arr in (u, u.astype(np.float64), oracle.bf16_from_f32(u)):
            np.testing.assert_array_equal(oracle.sign_pack(arr), expect, err_msg=case["name"])


@pytest.mark.parametrize("n", [1, 63, 64, 65, 1000, 4096])
def test_pack_roundtrip_against_numpy_unpackbits(n):
    u = synthetic.random_matrix(70 + n, (n,))
    words = oracle.sign_pack(u)
    assert words.size == (n + 63) // 64
    bits = np.unpackbits(words.view(np.uint8), bitorder="little")
    np.testing.assert_array_equal(bits[:n], (u >= 0).astype(np.uint8))
    assert not bits[n:].any()  # zero tail


def test_payload_is_one_bit_per_entry(golden_dir):
    spec = json.load(open(os.path.join(golden_dir, "payload_ratio.json")))
    for (R, C) in synthetic.WORKLOADS["gpt2s_mw8_k1"].shapes[:4]:
        n = R * C
        words = oracle.sign_pack(np.ones(n, np.float32))
        assert words.nbytes * 8 == n * spec["bits_per_param_packed"]
        assert (4 * n) // words.nbytes == spec["reduction_vs_fp32_packed"]
        assert (4 * n) // (n * spec["bits_per_param_int8"] // 8) == spec["reduction_vs_fp32_int8"]


# ---------------------------------------------------------------------------
# O6 + O7 vote and update
# ---------------------------------------------------------------------------
def _pack_bits(bits):
    """bits: [mw][n] of 0/1 -> [mw][words] uint64 via numpy packbits."""
    mw, n = bits.shape
    nw = (n + 63) // 64
    padded = np.zeros((mw, nw * 64), np.uint8)
    padded[:, :n] = bits
    return np.packbits(padded, axis=1, bitorder="little").view(np.uint64).reshape(mw, nw)


@pytest.mark.parametrize("mw", [1, 2, 3, 4])
def test_vote_exhaustive_small_worker_counts(mw):
    n = 1 << mw
    e = np.arange(n)
    bits = np.array([(e >> m) & 1 for m in range(mw)], np.uint8)
    w = np.zeros(n, np.float32)
    vote = oracle.vote_update(_pack_bits(bits), w, 0.25)
    for i in range(n):
        plus = bin(i).count("1")
        expect = 1 if 2 * plus > mw else (-1 if 2 * plus < mw else 0)
        assert vote[i] == expect
        assert w[i] == -0.25 * expect


def test_vote_worked_example_from_pages(golden_dir):
    spec = json.load(open(os.path.join(golden_dir, "vote_worked_example.json")))
    for case in spec["cases"]:
        mw, plus = case["workers"], case["plus_votes"]
        bits = np.zeros((mw, 1), np.uint8)
        bits[:plus, 0] = 1
        w = np.zeros(1, np.float32)
        vote = oracle.vote_update(_pack_bits(bits), w, 1.0)
        assert vote[0] == case["expected_vote"]


@pytest.mark.parametrize("mw", [5, 7, 8, 15, 16])
def test_vote_random_against_counting(mw):
    rng = np.random.default_rng(mw)
    n = 3001
    bits = rng.integers(0, 2, (mw, n)).astype(np.uint8)
    packed = _pack_bits(bits)
    w0 = rng.standard_normal(n).astype(np.float32)
    w = w0.copy()
    vote = oracle.vote_update(packed, w, 1e-3)
    total = bits.astype(np.int64).sum(0) * 2 - mw
    np.testing.assert_array_equal(vote, np.sign(total))
    if mw % 2:
        assert (vote != 0).all()
    eta = np.float32(1e-3)
    expect = np.where(vote > 0, w0 - eta, np.where(vote < 0, w0 + eta, w0)).astype(np.float32)
    np.testing.assert_array_equal(w, expect)
    # worker order does not matter
    w2 = w0.copy()
    vote2 = oracle.vote_update(packed[rng.permutation(mw)], w2, 1e-3)
    np.testing.assert_array_equal(vote2, vote)
    np.testing.assert_array_equal(w2, w)


# ---------------------------------------------------------------------------
# spectral normalisation (summary §4 "nanoGPT": spectral as well as
# Frobenius scaling): power iteration on the Gram matrix
# ---------------------------------------------------------------------------
def _psd(rng, r, c):
    m = rng.standard_normal((r, c))
    return m @ m.T


@pytest.mark.parametrize("r,c", [(8, 20), (16, 16), (5, 40)])
def test_power_lambda_below_top_eigenvalue_and_nondecreasing(r, c):
    a = _psd(np.random.default_rng(r * c), r, c)
    top = np.linalg.eigvalsh(a)[-1]
    prev = 0.0
    for p in (1, 2, 3, 5, 10, 30):
        lam = oracle.power_lambda(a, p)
        assert lam <= top * (1 + 1e-12)
        assert lam >= prev * (1 - 1e-12)
        prev = lam


def test_power_lambda_converges_to_top_eigenvalue():
    rng = np.random.default_rng(3)
    q, _ = np.linalg.qr(rng.standard_normal((12, 12)))
    d = np.linspace(1.0, 3.0, 12)
    d[-1] = 6.0  # a clear gap
    a = (q * d) @ q.T
    assert oracle.power_lambda(a, 400) == pytest.approx(6.0, rel=1e-12)


def test_power_lambda_rank_one_is_exact_after_two_steps():
    rng = np.random.default_rng(4)
    v = rng.standard_normal(9)
    a = np.outer(v, v)
    assert oracle.power_lambda(a, 2) == pytest.approx(float(v @ v), rel=1e-13)


def test_power_lambda_diagonal_closed_form():
    """From the all-ones start, the p-th step's ||A v|| on A = diag(d) is
    sqrt(sum d^(2p)) / sqrt(sum d^(2p-2))."""
    d = np.array([0.5, 1.0, 2.0, 3.0, 3.5], np.float64)
    for p in (1, 2, 4, 7):
        expect = math.sqrt(float(np.sum(d ** (2 * p)))) / math.sqrt(float(np.sum(d ** (2 * p - 2))))
        assert oracle.power_lambda(np.diag(d), p) == pytest.approx(expect, rel=1e-13)


@pytest.mark.parametrize("shape", [(6, 10), (10, 6), (8, 8)])
@pytest.mark.parametrize("k", [0, 1, 2, 5])
def test_spectral_ns_is_the_cubic_on_sigma_over_sigma_max(shape, k):
    """Exact mode, converged power iteration: X_k = U p^k(S / s_max) V^T (SVD
    from numpy), so the top singular value is 1 for every k."""
    R, C = shape
    rng = np.random.default_rng(R * 100 + C + k)
    u_, _, vt = np.linalg.svd(rng.standard_normal((R, C)), full_matrices=False)
    sig = np.linspace(0.3, 1.0, min(R, C)) * 2.5
    sig[0] = 4.0  # gap so that 300 steps converge
    m = (u_ * sig) @ vt
    lam, x0, a0 = oracle.spectral_x0_a0(m, oracle.F64, 300)
    assert lam == pytest.approx(16.0, rel=1e-12)
    x = oracle.newton_schulz_a0(x0, a0, k, oracle.F64)
    expect = (u_ * scalar_map(sig / 4.0, k)) @ vt
    assert rel_fro(x, expect) < 1e-10
    assert np.linalg.svd(x, compute_uv=False)[0] == pytest.approx(1.0, abs=1e-10)


@pytest.mark.parametrize("mode", [F32, BF16])
def test_spectral_power_of_two_scale_invariance_exact(mode):
    rng = np.random.default_rng(21)
    m = rng.standard_normal((24, 40)).astype(np.float32)
    if mode == BF16:
        m = oracle.bf16_from_f32(m)
        m4 = oracle.bf16_from_f32(oracle.bf16_to_f32(m) * np.float32(4.0))
    else:
        m4 = m * np.float32(4.0)
    l1, x1, a1 = oracle.spectral_x0_a0(m, mode, 6)
    l4, x4, a4 = oracle.spectral_x0_a0(m4, mode, 6)
    assert l4 == 16.0 * l1
    np.testing.assert_array_equal(a1, a4)
    np.testing.assert_array_equal(x1, x4)
    np.testing.assert_array_equal(oracle.newton_schulz_a0(x1, a1, 3, mode),
                                  oracle.newton_schulz_a0(x4, a4, 3, mode))


def test_spectral_k0_is_m_over_sigma_hat():
    rng = np.random.default_rng(22)
    m = rng.standard_normal((12, 30)).astype(np.float32)
    lam, x0, _ = oracle.spectral_x0_a0(m, F32, 5)
    np.testing.assert_allclose(x0, m.astype(np.float64) / math.sqrt(lam), rtol=1e-15)


def test_spectral_equals_frobenius_on_rank_one_momentum():
    """Rank one: ||M||_F = ||M||_2, and power iteration is exact after two
    steps, so both normalisations give the same iterate (exact mode)."""
    rng = np.random.default_rng(23)
    m = np.outer(rng.standard_normal(7), rng.standard_normal(11))
    _, x0f = oracle.normalise(m)
    _, x0s, a0 = oracle.spectral_x0_a0(m, oracle.F64, 2)
    assert rel_fro(x0s, x0f) < 1e-14
    assert rel_fro(oracle.newton_schulz_a0(x0s, a0, 3, oracle.F64),
                   oracle.newton_schulz(x0f, 3, oracle.F64)) < 1e-13


def test_step_spectral_matches_its_parts():
    """The step with spectral normalisation is momentum, spectral scaling,
    Newton-Schulz, sign, vote: assembled here from the separately pinned
    parts."""
    rng = np.random.default_rng(24)
    mw, R, C = 3, 16, 24
    g = rng.standard_normal((mw, R, C)).astype(np.float32)
    m = np.zeros((mw, R, C), np.float32)
    w0 = rng.standard_normal((R, C)).astype(np.float32)
    w = w0.copy()
    packed, vote, u = oracle.step_matrix(g, m.copy(), w, 0.9, 1e-3, 2, F32, want_u=True,
                                         norm=oracle.NORM_SPECTRAL, power_iters=4)
    m_ref = m.copy()
    oracle.momentum(g, m_ref, 0.9)
    pk = []
    for j in range(mw):
        _, x0, a0 = oracle.spectral_x0_a0(m_ref[j], F32, 4)
        uj = oracle.newton_schulz_a0(x0, a0, 2, F32)
        np.testing.assert_array_equal(u[j], uj)
        pk.append(oracle.sign_pack(uj))
    np.testing.assert_array_equal(packed, np.stack(pk))
    w_ref = w0.copy()
    np.testing.assert_array_equal(vote, oracle.vote_update(np.stack(pk), w_ref, 1e-3))
    np.testing.assert_array_equal(w, w_ref)


# ---------------------------------------------------------------------------
# int8 payload: the vote as the sign of the integer sum of the workers' signs
# (summary §2 "Core mechanism" and "Communication efficiency")
# ---------------------------------------------------------------------------
def test_int8_signs_follow_the_packed_rule():
    rng = np.random.default_rng(31)
    u = rng.standard_normal(1000).astype(np.float32)
    u[:4] = [0.0, -0.0, np.nan, -np.inf]
    s = oracle.sign_int8(u)
    bits = np.unpackbits(oracle.sign_pack(u).view(np.uint8), bitorder="little")[:u.size]
    np.testing.assert_array_equal(s, 2 * bits.astype(np.int8) - 1)
    assert set(np.unique(s)) <= {-1, 1}


def test_int8_payload_is_eight_bits_per_entry(golden_dir):
    spec = json.load(open(os.path.join(golden_dir, "payload_ratio.json")))
    n = 4096
    s = oracle.sign_int8(np.ones(n, np.float32))
    assert s.nbytes * 8 == spec["bits_per_param_int8"] * n
    assert 32 // spec["bits_per_param_int8"] == spec["reduction_vs_fp32_int8"]


@pytest.mark.parametrize("mw", [1, 2, 3, 4, 5, 8, 10, 16, 17])
def test_int8_vote_equals_packed_vote(mw):
    """Two formulations of the same vote: the integer sum of +-1 values and
    the count of set bits."""
    rng = np.random.default_rng(100 + mw)
    n = 2049
    u = rng.standard_normal((mw, n)).astype(np.float32)
    u[:, :7] = 0.0  # ties of +0 values and (even mw) tied votes
    packed = np.stack([oracle.sign_pack(u[m]) for m in range(mw)])
    signs = np.stack([oracle.sign_int8(u[m]) for m in range(mw)])
    w0 = rng.standard_normal(n).astype(np.float32)
    w_a, w_b = w0.copy(), w0.copy()
    v_a = oracle.vote_update(packed, w_a, 1e-3)
    v_b = oracle.vote_update_int8(signs, w_b, 1e-3)
    np.testing.assert_array_equal(v_a, v_b)
    np.testing.assert_array_equal(w_a.view(np.uint32), w_b.view(np.uint32))


def test_int8_vote_brute_force_general_values():
    """The sum is the plain integer sum of the int8 values (any value, not
    only +-1): checked entry by entry in Python."""
    rng = np.random.default_rng(5)
    mw, n = 6, 300
    signs = rng.integers(-128, 128, (mw, n)).astype(np.int8)
    signs[:, :5] = 0
    w0 = rng.standard_normal(n).astype(np.float32)
    w = w0.copy()
    vote = oracle.vote_update_int8(signs, w, 0.5)
    for i in range(n):
        total = sum(int(signs[m, i]) for m in range(mw))
        expect = (total > 0) - (total < 0)
        assert vote[i] == expect
        assert w[i] == np.float32(w0[i] - np.float32(0.5) * expect)


def test_int8_vote_worked_example_from_pages(golden_dir):
    spec = json.load(open(os.path.join(golden_dir, "vote_worked_example.json")))
    for case in spec["cases"]:
        mw, plus = case["workers"], case["plus_votes"]
        signs = -np.ones((mw, 1), np.int8)
        signs[:plus, 0] = 1
        w = np.zeros(1, np.float32)
        assert oracle.vote_update_int8(signs, w, 1.0)[0] == case["expected_vote"]


def test_update_moves_exactly_eta_on_dyadic_grid():
    rng = np.random.default_rng(9)
    n = 5000
    w0 = (rng.integers(-(1 << 19), 1 << 19, n) * 2.0 ** -20).astype(np.float32)
    bits = rng.integers(0, 2, (4, n)).astype(np.uint8)
    w = w0.copy()
    eta = 2.0 ** -10
    vote = oracle.vote_update(_pack_bits(bits), w, eta)
    delta = w.astype(np.float64) - w0.astype(np.float64)
    assert set(np.unique(delta)) <= {-eta, 0.0, eta}
    np.testing.assert_array_equal(delta, -eta * vote)


# ---------------------------------------------------------------------------
# whole step: special cases that reduce to textbook methods
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("mom", ["f32", "bf16"])
def test_step_k0_is_majority_vote_signum(mom):
    """k = 0 leaves U = M'/||M'||, so the step is the majority vote of the
    momentum signs (majority-vote signSGD with momentum); from M0 = 0 the
    momentum equals the gradient, whose sign storage rounding keeps."""
    mw, R, C = 5, 9, 20
    g = np.stack([synthetic.random_matrix(300 + i, (R, C)) for i in range(mw)])
    m = np.zeros((mw, R, C), np.float32 if mom == "f32" else np.uint16)
    w0 = synthetic.random_matrix(400, (R, C), 0.02)
    w = w0.copy()
    packed, vote, _ = oracle.step_matrix(g, m, w, 0.9, 1e-3, 0, BF16 if mom == "bf16" else F32)
    plus = (g >= 0).sum(0)
    np.testing.assert_array_equal(vote, np.sign(2 * plus - mw))
    eta = np.float32(1e-3)
    np.testing.assert_array_equal(w, np.where(vote > 0, w0 - eta, w0 + eta))


def test_step_single_worker_is_sign_of_polar_direction():
    """Mw = 1: the vote is the worker's own sign of its polar direction,
    checked here against numpy's SVD polar factor at large k."""
    R, C = 7, 12
    g = synthetic.random_matrix(500, (1, R, C))
    m = np.zeros((1, R, C), np.float32)
    w0 = synthetic.random_matrix(501, (R, C), 0.02)
    w = w0.copy()
    _, vote, u = oracle.step_matrix(g, m, w, 0.9, 1e-3, 60, F64, want_u=True)
    us, _, vt = np.linalg.svd(g[0].astype(np.float64), full_matrices=False)
    polar = us @ vt
    keep = np.abs(polar) > 1e-9
    np.testing.assert_array_equal(vote[keep], np.where(polar[keep] >= 0, 1, -1))


def test_step_two_steps_keep_momentum_state():
    """The momentum buffer is the only state: two steps equal step 1, a copy
    of (M, W), then step 2 on the copy."""
    mw, R, C = 3, 6, 10
    g1 = np.stack([synthetic.random_matrix(600 + i, (R, C)) for i in range(mw)])
    g2 = np.stack([synthetic.random_matrix(700 + i, (R, C)) for i in range(mw)])
    m = np.zeros((mw, R, C), np.uint16)
    w = synthetic.random_matrix(800, (R, C), 0.02)
    oracle.step_matrix(g1, m, w, 0.9, 1e-3, 2, BF16)
    m_saved, w_saved = m.copy(), w.copy()
    p_a, v_a, _ = oracle.step_matrix(g2, m, w, 0.9, 1e-3, 2, BF16)
    p_b, v_b, _ = oracle.step_matrix(g2, m_saved, w_saved, 0.9, 1e-3, 2, BF16)
    np.testing.assert_array_equal(m, m_saved)
    np.testing.assert_array_equal(w, w_saved)
    np.testing.assert_array_equal(p_a, p_b)
    # and the second momentum is the fma of the first
    m1 = np.zeros((mw, R, C), np.uint16)
    oracle.momentum(g1, m1, 0.9)
    m1_vals = oracle.bf16_to_f32(m1).ravel()
    g2f = g2.ravel()
    ref = np.array([exact_round_f32(Fraction(float(np.float32(0.9))) * Fraction(float(a))
                                    + Fraction(float(b))) for a, b in zip(m1_vals, g2f)],
                   np.float32)
    np.testing.assert_array_equal(m.ravel(), torch_bf16_bits(ref))


# ---------------------------------------------------------------------------
# O8 post-vote polar step
# ---------------------------------------------------------------------------
def test_post_polar_zero_vote_is_noop():
    w = synthetic.random_matrix(900, (5, 7))
    w0 = w.copy()
    assert oracle.post_polar(np.zeros((5, 7), np.int8), w, 1e-3, 5, BF16) == 0
    np.testing.assert_array_equal(w, w0)


@pytest.mark.parametrize("mode,shape", [(F64, (6, 10)), (F32, (4, 16)), (BF16, (4, 16)),
                                        (BF16, (16, 4))])
def test_post_polar_rank_one_vote_is_fixed_point(mode, shape):
    """An all-(+1) vote is rank one: V/||V||_F has singular value 1 and stays
    put, so W moves by -eta/sqrt(n) in one fused multiply-add. With stored
    iterates the 4x16 case keeps every intermediate a power of two."""
    R, C = shape
    n = R * C
    w = synthetic.random_matrix(901, (R, C), 0.02)
    w0 = w.copy()
    vote = np.ones((R, C), np.int8)
    assert oracle.post_polar(vote, w, 1e-3, 3, mode) == n
    y = np.float32(1.0 / math.sqrt(n))
    eta = np.float32(1e-3)
    expect = np.array([exact_round_f32(-Fraction(float(eta)) * Fraction(float(y))
                                       + Fraction(float(x))) for x in w0.ravel()], np.float32)
    np.testing.assert_array_equal(w.ravel(), expect)


def test_post_polar_signed_permutation_vote():
    R, C, k = 4, 9, 2
    vote = signed_partial_permutation(R, C, seed=3).astype(np.int8)
    w = np.zeros((R, C), np.float32)
    assert oracle.post_polar(vote, w, 1.0, k, F64) == R
    x = 0.5
    for _ in range(k):
        x = 1.5 * x - 0.5 * (x * x) * x
    np.testing.assert_array_equal(w, (-np.float32(x) * vote).astype(np.float32))


# ---------------------------------------------------------------------------
# the workload table (shapes of the pages' models)
# ---------------------------------------------------------------------------
def test_workload_shapes():
    gpt = synthetic.WORKLOADS["gpt2s_mw8_k1"]
    assert len(gpt.shapes) == 48 and gpt.params == 84_934_656
    assert abs(gpt.ns_flops() - 1.566e12) / 1.566e12 < 1e-3
    res = synthetic.WORKLOADS["resnet50_all_convs_mw4_k1"]
    assert len(res.shapes) == 53 and res.params == 23_454_912
    blk = synthetic.WORKLOADS["block4096_mw16_k5"]
    assert blk.params == 157_286_400


def test_generators_are_seeded_and_distinct():
    wl = synthetic.WORKLOADS["square256_mw4_k1"]
    a = synthetic.gradient(wl, 0, 1, 0)
    np.testing.assert_array_equal(a, synthetic.gradient(wl, 0, 1, 0))
    assert not np.array_equal(a, synthetic.gradient(wl, 0, 2, 0))
    assert not np.array_equal(a, synthetic.gradient(wl, 0, 1, 1))
    assert a.dtype == np.float32 and a.shape == (256, 256)


# ---------------------------------------------------------------------------
# full-precision Muon step (the comparison point of the summary, one worker,
# no sign): U = NS(M / ||M||), W <- fmaf(-eta, U, W)
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("shape", [(6, 10), (10, 6), (8, 8)])
@pytest.mark.parametrize("k", [1, 3])
def test_muon_step_direction_is_the_svd_closed_form(shape, k):
    R, C = shape
    rng = np.random.default_rng(R * 31 + C + k)
    g = rng.standard_normal((R, C)).astype(np.float32)
    m = np.zeros((R, C), np.float32)
    w = np.zeros((R, C), np.float32)
    u = oracle.muon_step_matrix(g, m, w, 0.9, 1e-3, k, oracle.F64, want_u=True)
    np.testing.assert_array_equal(m, g)  # first step from M_0 = 0
    us, sig, vt = np.linalg.svd(g.astype(np.float64), full_matrices=False)
    expect = (us * scalar_map(sig / np.linalg.norm(sig), k)) @ vt
    assert rel_fro(u, expect) < 1e-12


def test_muon_step_update_is_one_fused_multiply_add():
    """W_new = fp32(-eta * fp32(U) + W_old), the product and sum exact before
    the one rounding (checked with exact rationals)."""
    rng = np.random.default_rng(32)
    R, C = 7, 9
    g = rng.standard_normal((R, C)).astype(np.float32)
    w0 = rng.standard_normal((R, C)).astype(np.float32)
    w = w0.copy()
    eta = np.float32(0.3)
    u = oracle.muon_step_matrix(g, np.zeros((R, C), np.float32), w, 0.9, float(eta), 2, F32,
                                want_u=True)
    u32 = u.astype(np.float32)
    for i in range(R):
        for j in range(C):
            q = -Fraction(float(eta)) * Fraction(float(u32[i, j])) + Fraction(float(w0[i, j]))
            assert w[i, j] == exact_round_f32(q)


def test_muon_step_rank_one_momentum_is_a_fixed_point():
    rng = np.random.default_rng(33)
    a, b = rng.integers(-3, 4, 7), rng.integers(-3, 4, 11)
    a[0], b[0] = 1, 2
    g = np.outer(a, b).astype(np.float32)  # exact in fp32
    for k in (1, 4):
        u = oracle.muon_step_matrix(g, np.zeros_like(g), np.zeros_like(g), 0.9, 1e-3, k,
                                    oracle.F64, want_u=True)
        assert rel_fro(u, g / np.linalg.norm(g.astype(np.float64))) < 1e-13


def test_single_worker_sign_muon_moves_by_eta_times_the_sign_of_the_muon_direction():
    rng = np.random.default_rng(34)
    R, C = 12, 20
    g = rng.standard_normal((R, C)).astype(np.float32)
    w = np.zeros((R, C), np.float32)
    u = oracle.muon_step_matrix(g, np.zeros((R, C), np.float32), w.copy(), 0.9, 1e-3, 2, F32,
                                want_u=True)
    w_sign = np.zeros((R, C), np.float32)
    oracle.step_matrix(g[None], np.zeros((1, R, C), np.float32), w_sign, 0.9, 1e-3, 2, F32)
    np.testing.assert_array_equal(w_sign, np.where(u >= 0, np.float32(-1e-3), np.float32(1e-3)))
