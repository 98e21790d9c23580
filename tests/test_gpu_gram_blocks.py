"""The bf16 Gram matrix A = X X^T of the first Newton-Schulz iteration
(pages: "Algorithmic flow", step 1, the cubic iteration on the smaller Gram
matrix), checked entry by entry on shapes that exercise every kind of tile of
the persistent Gram walk.

The walk covers A's upper triangle in 64 x 64 blocks, each stored with its
mirror: cross tiles take the blocks between two 256-row groups, and pair or
single tiles the blocks inside a group. A wrong, missing, misplaced or
transposed block would hardly move U as a whole (for random data an
off-diagonal Gram entry is about c^-1/2 of a diagonal one, below the effect of
A's own bf16 rounding on U), so this test recovers the A that the GPU applied
from U at k = 1. With X = M / ||M||_F (M the bf16 momentum, exactly
representable), U = 1.5 X - 0.5 A X, so A = (3 X - 2 U) X^T (X X^T)^-1, in
fp64. Every entry is compared with the definition X X^T (fp64):

  |A_gpu - X X^T| <= 2^-8 |X X^T| + tau (|X| |X|^T),
  tau = 2^-16 + 32 u r^1.5 / sqrt(c),   u = 2^-24.

The first term covers the single bf16 rounding of A (at most 2^-9 relative)
twice over; 2^-16 in tau covers the fp32 accumulation of the c products of
an entry (the probabilistic bound lambda sqrt(c/2) u sum|x x| with lambda = 4
is below 2^-17 sum|x x| here). The rest of tau is the recovery's own error:
the product accumulates A X - 3 X in fp32 at the magnitude of 3 X, so A X,
a correction of relative size ~1/r next to 3 X, carries an error of about
sqrt(r) u |x| per entry, and mapping it through X^+ (about r X^T for these
random X) gives about u r^1.5 c^-1/2 sum|x x| per entry of A; the maximum
over the r^2 entries of a matrix measured 12 times that at r = 1536,
c = 3072, so the factor 32 leaves room. Entries that a misplaced, missing or
transposed block would change are of the size of the off-diagonal Gram
entries, about sum|x x| / sqrt(c), 13 times tau sum|x x| or more on every
shape here: the test plants such mistakes in the recovered A (on the host)
and requires them to fail by a wide margin.

Shapes (wide and tall, two workers, every matrix in one launch): 1 group
(ragged and whole), 2 groups (ragged), 3 groups (pair tiles; whole, and a
last group of 8 rows), 4 groups (pair, single and cross tiles; whole and
ragged), 5 and 6 groups."""
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

import oracle
import sign_muon_step_amd as sm
import synthetic
from gpu_util import DEV, announce, make_matrix, run, to_host

pytestmark = pytest.mark.gpu

POOL = ThreadPoolExecutor(max_workers=8)

# every shape takes the walk: C % 8 == 0, min(R, C) % 8 == 0, and
# ceil(max(R, C) / 32) a multiple of 4 and at least 8
SHAPES = [(200, 512), (256, 640), (448, 1024), (520, 1280), (768, 1536), (1536, 768), (1024, 2048),
          (2048, 1000), (1000, 1920), (1280, 2560), (1536, 3072)]
MW = 2


@pytest.fixture(autouse=True)
def _name_the_case(request):
    announce(f"[gpu-test] {request.node.nodeid}")
    yield
    torch.cuda.synchronize()


def implied_gram(u, m):
    """(A as the GPU applied it, X X^T, the per-entry bound) for one worker's
    U and bf16 momentum M, in the Gram's r x c orientation."""
    tall = m.shape[0] > m.shape[1]
    _, x = oracle.normalise(m)
    x = x.astype(np.float64)
    u = u.astype(np.float64)
    if tall:
        x, u = x.T, u.T
    r, c = x.shape
    gram = x @ x.T
    a_gpu = ((3.0 * x - 2.0 * u) @ x.T) @ np.linalg.inv(gram)
    tau = 2.0 ** -16 + 32 * 2.0 ** -24 * r ** 1.5 / np.sqrt(c)
    bound = 2.0 ** -8 * np.abs(gram) + tau * (np.abs(x) @ np.abs(x).T)
    return a_gpu, gram, bound


def worst(a, gram, bound):
    ratio = np.abs(a - gram) / bound
    i, l = np.unravel_index(int(np.argmax(ratio)), ratio.shape)
    return float(ratio[i, l]), (int(i), int(l))


def planted(a):
    """Copies of a with one block transposed, one block zeroed and one block
    taken from its neighbour (64 x 64 blocks off the diagonal)."""
    t, z, s = a.copy(), a.copy(), a.copy()
    t[0:64, 64:128] = a[0:64, 64:128].T
    z[64:128, 128:192] = 0.0
    s[0:64, 128:192] = a[0:64, 64:128]
    return t, z, s


def test_gram_walk_blocks_entry_by_entry():
    def grads(j):
        return np.stack([synthetic.random_matrix(4400 + 10 * j + w, SHAPES[j], 1e-3) for w in range(MW)])

    g = list(POOL.map(grads, range(len(SHAPES))))
    mats = [make_matrix(g[j], np.zeros((MW,) + s, np.uint16), vote=False, packed=False)
            for j, s in enumerate(SHAPES)]
    p = sm.Params(workers=MW, beta=0.9, eta=1e-3, ns_iters=1, mom_dtype=sm.BF16, ns_dtype=sm.BF16)
    announce(f"  {len(SHAPES)} matrices, {MW} workers, k = 1: momentum + Newton-Schulz, U stored")
    run("signmuon_momentum_ns", mats, p)
    cases = [(j, w) for j in range(len(SHAPES)) for w in range(MW)]

    def check(jw):
        j, w = jw
        m = to_host(mats[j].momentum)[w]
        m_ref = np.zeros(SHAPES[j], np.uint16)
        oracle.momentum(g[j][w], m_ref, 0.9)
        np.testing.assert_array_equal(m, m_ref)
        a, gram, bound = implied_gram(to_host(mats[j].polar_out)[w], m_ref)
        return worst(a, gram, bound), min(worst(b, gram, bound)[0] for b in planted(a))

    top = 0.0
    for (j, w), ((ratio, at), plant) in zip(cases, POOL.map(check, cases)):
        announce(f"  {SHAPES[j]} worker {w}: max |dA| / bound = {ratio:.3f} at {at}; "
                 f"planted block mistakes: at least {plant:.1f}")
        top = max(top, ratio)
        assert plant >= 4.0, "the check must see a wrong block"
    assert top <= 1.0
