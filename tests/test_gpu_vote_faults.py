"""The majority vote with a faulty or a missing worker, on the GPU through the
C ABI, bit-exact against the oracle (O6+O7).

The summary's §5 "Significance" names robustness to individual workers as a
property of the sign-majority aggregation. What a single worker can do to the
vote follows from the counting rule alone: with c the number of +1 signs
among Mw workers, the vote is sign(2c - Mw). One worker flipping its bit
moves 2c - Mw by 2, and removing one worker moves it by 1. So:
  - a worker forced to all +1 (all bits set) or all -1 (all bits clear)
    changes the vote only where |2c - Mw| <= 2, and only toward its own sign;
  - a vote over the Mw - 1 remaining buffers changes the full vote only where
    |2c - Mw| <= 1.
The GPU's vote and W on the faulty buffers must equal the oracle's bit for
bit, and the set of changed entries must obey these bounds (counted here by
brute force on the host)."""
import numpy as np
import pytest
import torch

import oracle
import sign_muon_step_amd as sm
from gpu_util import DEV, announce, to_dev, to_host

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _name_the_case(request):
    announce(f"[gpu-test] {request.node.nodeid}")
    yield
    torch.cuda.synchronize()


def random_packed(rng, mw, n):
    nw = (n + 63) // 64
    bits = rng.integers(0, 2, (mw, nw * 64), dtype=np.uint8)
    bits[:, n:] = 0
    return bits, np.packbits(bits, axis=1, bitorder="little").view(np.uint64).reshape(mw, nw)


def pack(bits):
    mw = bits.shape[0]
    return np.packbits(bits, axis=1, bitorder="little").view(np.uint64).reshape(mw, -1)


def gpu_vote(packed, n, w0, eta):
    w = to_dev(w0)
    vote = torch.zeros(n, dtype=torch.int8, device=DEV)
    sm.signmuon_vote_update(to_dev(np.ascontiguousarray(packed)), packed.shape[0], n, w, eta, vote)
    torch.cuda.synchronize()
    return to_host(vote), to_host(w)


def oracle_vote(packed, w0, eta):
    w = w0.copy()
    vote = oracle.vote_update(np.ascontiguousarray(packed), w, eta)
    return vote, w


@pytest.mark.parametrize("mw", [3, 4, 8, 9, 16, 17, 255])
@pytest.mark.parametrize("n", [4096 * 3 + 17, 100003])
@pytest.mark.parametrize("force", ["all_plus", "all_minus"])
def test_one_worker_forced(mw, n, force):
    rng = np.random.default_rng(mw * 31 + n % 1000 + (force == "all_plus"))
    bits, packed = random_packed(rng, mw, n)
    w0 = (rng.standard_normal(n) * 0.02).astype(np.float32)
    eta = 1e-3
    v_ok, _ = oracle_vote(packed, w0, eta)
    c = bits[:, :n].sum(axis=0).astype(np.int64)
    margin = np.abs(2 * c - mw)
    for f in (0, mw - 1):
        faulty = bits.copy()
        faulty[f, :n] = 1 if force == "all_plus" else 0
        fp = pack(faulty)
        v_gpu, w_gpu = gpu_vote(fp, n, w0, eta)
        v_ref, w_ref = oracle_vote(fp, w0, eta)
        np.testing.assert_array_equal(v_gpu, v_ref, err_msg=f"vote, worker {f} {force}")
        np.testing.assert_array_equal(w_gpu, w_ref, err_msg=f"W, worker {f} {force}")
        changed = v_gpu != v_ok
        announce(f"  Mw={mw} n={n} worker {f} {force}: {int(changed.sum())} of {n} votes changed, "
                 f"all with |2c - Mw| <= 2")
        assert (margin[changed] <= 2).all()
        toward = 1 if force == "all_plus" else -1
        assert (np.sign(v_gpu[changed].astype(int) - v_ok[changed].astype(int)) == toward).all()
        # entries far from a tie keep their vote and their W update
        far = margin > 2
        np.testing.assert_array_equal(v_gpu[far], v_ok[far])


@pytest.mark.parametrize("mw", [2, 3, 8, 9, 16, 255])
@pytest.mark.parametrize("n", [4096 * 2 + 33, 70001])
def test_vote_without_one_worker(mw, n):
    rng = np.random.default_rng(mw * 17 + n % 997)
    bits, packed = random_packed(rng, mw, n)
    w0 = (rng.standard_normal(n) * 0.02).astype(np.float32)
    eta = 2.0 ** -10
    v_full, _ = oracle_vote(packed, w0, eta)
    c = bits[:, :n].sum(axis=0).astype(np.int64)
    margin = np.abs(2 * c - mw)
    for f in (0, mw // 2, mw - 1):
        rest = np.delete(packed, f, axis=0)
        v_gpu, w_gpu = gpu_vote(rest, n, w0, eta)
        v_ref, w_ref = oracle_vote(rest, w0, eta)
        np.testing.assert_array_equal(v_gpu, v_ref, err_msg=f"vote without worker {f}")
        np.testing.assert_array_equal(w_gpu, w_ref, err_msg=f"W without worker {f}")
        changed = v_gpu != v_full
        announce(f"  Mw={mw} n={n} without worker {f}: {int(changed.sum())} of {n} votes changed")
        assert (margin[changed] <= 1).all()
