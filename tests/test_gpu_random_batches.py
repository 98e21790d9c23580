"""Seeded random batches through the whole step, against the oracle.

Each case draws (from a fixed seed) one to four matrices of random shape --
multiples of 8 or arbitrary sizes from 2 to 1099, wide and tall -- with one
to six workers, k in {0, 1, 2}, fp32 or bf16 Newton-Schulz, and Frobenius or
spectral scaling (1 to 8 power steps). The large cases take 8 to 16
matrices of 64 to 1032 rows and columns (multiples of 8) with 8 to 16
workers, so that the one-launch power iteration, the persistent walks and
the split-k Gram meet in one call. Every case runs signmuon_step with U
stored and checks, for the first and last worker of every matrix:
  - U against the oracle (k = 0: the scaled momentum, relative Frobenius
    error <= 1e-5; k >= 1: the whole Newton-Schulz result, <= 1e-5 in fp32
    and 2e-2 in bf16), with >= 99.9 % sign agreement on the entries with
    |U| >= 1e-6 max|U|;
  - the packed words equal the oracle's packing of the stored U.

A third test draws whole steps with every output: the packed-bit or int8
payload, U stored or not (without it the bf16 final products take the
persistent walk), and with the packed payload sometimes the post-vote polar
step. Its signs must agree with the oracle's U on >= 99.9 % of the entries
(every worker's signs equal the rule applied to its stored U when U is
stored), the vote and W must equal the oracle's vote and update of the GPU's
signs bit for bit, and with the polar step, under which W moves only by
-eta Y, W must lie within eta * 1.5 * tolerance * ||Y||_F (plus a few fp32
roundings of W) of the oracle's."""
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

import oracle
import sign_muon_step_amd as sm
import synthetic
from gpu_util import DEV, announce, bit_sign_stats, rel_fro, sign_stats, to_dev, to_host

pytestmark = pytest.mark.gpu

POOL = ThreadPoolExecutor(max_workers=12)
NS_TOL = {"f32": 1e-5, "bf16": 2e-2}


@pytest.fixture(autouse=True)
def _name_the_case(request):
    announce(f"[gpu-test] {request.node.nodeid}")
    yield
    torch.cuda.synchronize()


def draw_case(rng, case, big):
    ns = ("f32", "bf16")[case % 2]
    spectral = (case // 2) % 2 == 1
    k = int(rng.integers(0, 3))
    mw = int(rng.integers(8, 17)) if big else int(rng.integers(1, 7))
    nm = int(rng.integers(8, 17)) if big else int(rng.integers(1, 5))
    shapes = []
    for _ in range(nm):
        if big:
            shapes.append((int(rng.integers(8, 130)) * 8, int(rng.integers(8, 130)) * 8))
        else:
            dims = [int(rng.integers(1, 140)) * 8 if rng.random() < 0.6 else int(rng.integers(2, 1100))
                    for _ in range(2)]
            shapes.append(tuple(dims))
    power = int(rng.integers(1, 9)) if spectral else 0
    return ns, spectral, k, mw, shapes, power


def run_case(seed, case, big):
    rng = np.random.default_rng([seed, case])
    ns, spectral, k, mw, shapes, power = draw_case(rng, case, big)
    np_m = np.float32 if ns == "f32" else np.uint16
    code = sm.F32 if ns == "f32" else sm.BF16
    odt = oracle.F32 if ns == "f32" else oracle.BF16
    label = f"spectral p = {power}" if spectral else "frobenius"
    announce(f"  case {case}: {ns}, {label}, k = {k}, {mw} workers, shapes {shapes}")
    grads, mats = [], []
    for j, (R, C) in enumerate(shapes):
        g = np.stack([synthetic.random_matrix(seed * 100000 + case * 100 + 10 * j + w, (R, C), 1e-3)
                      for w in range(mw)])
        grads.append(g)
        mats.append(sm.Matrix(
            grad=to_dev(g), momentum=to_dev(np.zeros(g.shape, np_m)),
            packed=torch.zeros((mw, sm.signmuon_packed_words(R * C)), dtype=torch.int64, device=DEV),
            weight=to_dev(synthetic.random_matrix(seed * 100000 + case * 100 + 10 * j + 9, (R, C), 0.02)),
            polar_out=torch.zeros((mw, R, C), dtype=torch.float32, device=DEV),
            vote_out=torch.zeros((R, C), dtype=torch.int8, device=DEV)))
    p = sm.Params(workers=mw, beta=0.9, eta=1e-3, ns_iters=k, mom_dtype=code, ns_dtype=code,
                  norm=sm.NORM_SPECTRAL if spectral else sm.NORM_FROBENIUS, power_iters=power)
    sm.signmuon_step(mats, p, sm.workspace_tensor(mats, p, DEV))
    torch.cuda.synchronize()

    def reference(jw):
        j, w = jw
        m = np.zeros(shapes[j], np_m)
        oracle.momentum(grads[j][w], m, 0.9)
        if spectral:
            _, x0, a0 = oracle.spectral_x0_a0(m, odt, power)
            return x0 if k == 0 else oracle.newton_schulz_a0(x0, a0, k, odt)
        _, x0 = oracle.normalise(m)
        return x0 if k == 0 else oracle.newton_schulz(x0, k, odt)

    pairs = [(j, w) for j in range(len(shapes)) for w in sorted({0, mw - 1})]
    tol = NS_TOL[ns] if k > 0 else 1e-5
    worst = 0.0
    for (j, w), u_ref in zip(pairs, POOL.map(reference, pairs)):
        u = to_host(mats[j].polar_out)[w]
        np.testing.assert_array_equal(to_host(mats[j].packed)[w], oracle.sign_pack(u),
                                      err_msg=f"case {case} matrix {shapes[j]} worker {w}: packed")
        err = rel_fro(u, u_ref)
        agree, bad, n = sign_stats(u, u_ref)
        worst = max(worst, err / tol)
        assert err <= tol, f"case {case} matrix {shapes[j]} worker {w}: rel err {err:.3e}"
        assert agree >= 0.999, f"case {case} matrix {shapes[j]} worker {w}: {bad} of {n} signs differ"
    announce(f"    worst error / tolerance {worst:.3f}")


def test_random_small_batches():
    for case in range(48):
        run_case(41, case, big=False)


def test_random_large_batches():
    for case in range(6):
        run_case(43, case, big=True)


def run_whole_step(seed, case):
    rng = np.random.default_rng([seed, case])
    ns = ("f32", "bf16")[int(rng.integers(0, 2))]
    spectral = rng.random() < 0.4
    int8 = rng.random() < 0.4
    polar = rng.random() < 0.5
    k = int(rng.integers(0, 3))
    post = int(rng.integers(1, 3)) if (rng.random() < 0.3 and not int8) else 0
    mw = int(rng.integers(1, 10))
    shapes = [tuple(int(rng.integers(1, 130)) * 8 if rng.random() < 0.6 else int(rng.integers(2, 1000))
                    for _ in range(2)) for _ in range(int(rng.integers(1, 5)))]
    power = int(rng.integers(1, 9)) if spectral else 0
    np_m = np.float32 if ns == "f32" else np.uint16
    code = sm.F32 if ns == "f32" else sm.BF16
    odt = oracle.F32 if ns == "f32" else oracle.BF16
    eta = 1e-3
    announce(f"  case {case}: {ns}, {'spectral p = %d' % power if spectral else 'frobenius'}, k = {k}, "
             f"{mw} workers, {'int8' if int8 else 'packed'}, U {'stored' if polar else 'not stored'}, "
             f"polar step {post}, shapes {shapes}")
    grads, w0s, mats = [], [], []
    for j, (R, C) in enumerate(shapes):
        base = seed * 100000 + case * 100 + 10 * j
        g = np.stack([synthetic.random_matrix(base + w, (R, C), 1e-3) for w in range(mw)])
        w0 = synthetic.random_matrix(base + 9, (R, C), 0.02)
        grads.append(g)
        w0s.append(w0)
        mats.append(sm.Matrix(
            grad=to_dev(g), momentum=to_dev(np.zeros(g.shape, np_m)),
            packed=None if int8 else torch.zeros((mw, sm.signmuon_packed_words(R * C)), dtype=torch.int64,
                                                 device=DEV),
            weight=to_dev(w0),
            polar_out=torch.zeros((mw, R, C), dtype=torch.float32, device=DEV) if polar else None,
            vote_out=torch.zeros((R, C), dtype=torch.int8, device=DEV),
            signs_i8=torch.zeros((mw, R, C), dtype=torch.int8, device=DEV) if int8 else None))
    p = sm.Params(workers=mw, beta=0.9, eta=eta, ns_iters=k, mom_dtype=code, ns_dtype=code,
                  norm=sm.NORM_SPECTRAL if spectral else sm.NORM_FROBENIUS, power_iters=power,
                  payload=sm.PAYLOAD_INT8 if int8 else sm.PAYLOAD_BITS, post_polar_iters=post)
    sm.signmuon_step(mats, p, sm.workspace_tensor(mats, p, DEV))
    torch.cuda.synchronize()

    def reference(jw):
        j, w = jw
        m = np.zeros(shapes[j], np_m)
        oracle.momentum(grads[j][w], m, 0.9)
        if spectral:
            _, x0, a0 = oracle.spectral_x0_a0(m, odt, power)
            return x0 if k == 0 else oracle.newton_schulz_a0(x0, a0, k, odt)
        _, x0 = oracle.normalise(m)
        return x0 if k == 0 else oracle.newton_schulz(x0, k, odt)

    pairs = [(j, w) for j in range(len(shapes)) for w in sorted({0, mw - 1})]
    tol = NS_TOL[ns] if k > 0 else 1e-5
    for (j, w), u_ref in zip(pairs, POOL.map(reference, pairs)):
        where = f"case {case} matrix {shapes[j]} worker {w}"
        if polar:
            assert rel_fro(to_host(mats[j].polar_out)[w], u_ref) <= tol, f"{where}: U"
        if int8:
            agree, bad, n = sign_stats(to_host(mats[j].signs_i8)[w].astype(np.float64), u_ref)
        else:
            agree, bad, n = bit_sign_stats(to_host(mats[j].packed)[w], u_ref)
        assert agree >= 0.999, f"{where}: {bad} of {n} signs differ from the oracle's"
    for j in range(len(shapes)):
        where = f"case {case} matrix {shapes[j]}"
        signs = to_host(mats[j].signs_i8) if int8 else to_host(mats[j].packed)
        if polar:
            u = to_host(mats[j].polar_out)
            for w in range(mw):
                rule = oracle.sign_int8(u[w]) if int8 else oracle.sign_pack(u[w])
                np.testing.assert_array_equal(signs[w], rule, err_msg=f"{where} worker {w}: signs of U")
        w_ref = w0s[j].copy()
        vote = (oracle.vote_update_int8 if int8 else oracle.vote_update)(signs, w_ref, eta)
        np.testing.assert_array_equal(to_host(mats[j].vote_out), vote, err_msg=f"{where}: vote")
        w_gpu = to_host(mats[j].weight)
        if post == 0:
            np.testing.assert_array_equal(w_gpu, w_ref, err_msg=f"{where}: W")
        else:
            w_ref = w0s[j].copy()  # W moves only by the polar step of the vote
            oracle.post_polar(vote, w_ref, eta, post, odt)
            y_norm = np.linalg.norm((w0s[j].astype(np.float64) - w_ref) / eta)
            off = np.linalg.norm(w_gpu.astype(np.float64) - w_ref)
            bound = (eta * 1.5 * NS_TOL[ns] * y_norm
                     + 4 * np.sqrt(w_ref.size) * 2.0 ** -24 * float(np.abs(w_ref).max()))
            assert off <= bound, f"{where}: W after the polar step off by {off:.2e} (bound {bound:.2e})"


def test_random_whole_steps():
    for case in range(40):
        run_whole_step(47, case)
