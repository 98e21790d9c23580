"""GPU parity at the size limits the library accepts: a row or a column count
of 2^20 (the largest dimension), next to a small other side, so that the
Gram matrix stays tiny for the oracle while the kernels' long k loops,
64-bit offsets, ragged tiles and tails run at full length; and the worker
limit of the vote (255). Every step is compared with the oracle on the same
inputs: momentum, packed bits given U, vote and W bit-exact, U within the
Newton-Schulz tolerance.

The fp32 bound of the configured workloads (1e-5) assumes their contraction
lengths (c <= 11008). Here the Gram entries are fp32 sums of up to 2^20
terms, accumulated in order on the matrix cores, whose first-order worst-case
relative error is c * 2^-24; U inherits it (for k = 1 and a normalised X,
dU/U is about half of dA/A). The fp32 tolerance is therefore
max(1e-5, c * 2^-24); bf16 keeps 2e-2, which is larger."""
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

import oracle
import sign_muon_step_amd as sm
import synthetic
from gpu_util import DEV, announce, dtype_of, make_matrix, rel_fro, run, sign_stats, to_dev, to_host

pytestmark = pytest.mark.gpu

NS_TOL = {"f32": 1e-5, "bf16": 2e-2}
ORC_DT = {"f32": oracle.F32, "bf16": oracle.BF16}
POOL = ThreadPoolExecutor(max_workers=8)
MAX_DIM = 1 << 20


@pytest.fixture(autouse=True)
def _name_the_case(request):
    announce(f"[gpu-test] {request.node.nodeid}")
    yield
    torch.cuda.synchronize()


def one_step(shape, mw, k, ns, seed):
    R, C = shape
    np_m = dtype_of(ns)[0]
    g = np.stack([synthetic.random_matrix(seed * 100 + i, (R, C), 1e-3) for i in range(mw)])
    w0 = synthetic.random_matrix(seed * 100 + 99, (R, C), 0.02)
    mat = make_matrix(g, np.zeros((mw, R, C), np_m), w0)
    code = dtype_of(ns)[2]
    run("signmuon_step", [mat], sm.Params(workers=mw, beta=0.9, eta=1e-3, ns_iters=k,
                                          mom_dtype=code, ns_dtype=code))
    m_ref = np.zeros((mw, R, C), np_m)
    oracle.momentum(g, m_ref, 0.9)
    np.testing.assert_array_equal(to_host(mat.momentum), m_ref)
    u = to_host(mat.polar_out)
    packed = to_host(mat.packed)

    def ref(w):
        _, x0 = oracle.normalise(m_ref[w])
        return oracle.newton_schulz(x0, k, ORC_DT[ns])

    u_ref = list(POOL.map(ref, range(mw)))
    for w in range(mw):
        np.testing.assert_array_equal(packed[w], oracle.sign_pack(u[w]))
        err = rel_fro(u[w], u_ref[w])
        agree, bad, n = sign_stats(u[w], u_ref[w])
        announce(f"  {shape} {ns} k={k} worker {w}: rel err {err:.2e}, sign agreement {agree:.6f}"
                 f" ({bad} of {n} differ)")
        tol = max(NS_TOL[ns], max(R, C) * 2.0 ** -24)
        assert err <= tol
        assert agree >= 0.999
    w_ref = w0.copy()
    vote = oracle.vote_update(packed, w_ref, 1e-3)
    np.testing.assert_array_equal(to_host(mat.vote_out), vote)
    np.testing.assert_array_equal(to_host(mat.weight), w_ref)


@pytest.mark.parametrize("ns", ["f32", "bf16"])
@pytest.mark.parametrize("shape", [(1, MAX_DIM), (MAX_DIM, 1), (3, MAX_DIM - 5), (MAX_DIM - 3, 2)])
def test_longest_dimension(ns, shape):
    one_step(shape, 3, 1 if shape[0] != 3 else 2, ns, seed=shape[0] + shape[1] % 97)


def test_vote_at_the_worker_limit():
    """255 workers (the counters' 8 bit-planes), ragged n, k = 1."""
    mw, R, C = 255, 24, 40
    one_step((R, C), mw, 1, "f32", seed=31)
