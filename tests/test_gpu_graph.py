"""signmuon_step captured in a HIP graph: the library enqueues only kernel
launches on the caller's stream (no allocation, no memset, no host
synchronisation), so a captured step can be replayed (Frobenius and spectral
scaling). Two copies of the same
state advance side by side, one by graph replays and one by eager calls, with
eager work and synchronisations between the replays; after every replay the
momentum, the packed signs, the vote and W of both copies must be equal bit
for bit."""
import numpy as np
import pytest
import torch

import sign_muon_step_amd as sm
import synthetic
from gpu_util import DEV, announce, to_dev, to_host

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _name_the_case(request):
    announce(f"[gpu-test] {request.node.nodeid}")
    yield
    torch.cuda.synchronize()


def state(shapes, mw, seed, int8):
    mats = []
    for j, (R, C) in enumerate(shapes):
        g = np.stack([synthetic.random_matrix(seed + 10 * j + m, (R, C), 1e-3) for m in range(mw)])
        mats.append(sm.Matrix(
            grad=to_dev(g), momentum=torch.zeros((mw, R, C), dtype=torch.bfloat16, device=DEV),
            packed=None if int8 else torch.zeros((mw, sm.signmuon_packed_words(R * C)),
                                                 dtype=torch.int64, device=DEV),
            weight=to_dev(synthetic.random_matrix(seed + 10 * j + 9, (R, C), 0.02)),
            vote_out=torch.zeros((R, C), dtype=torch.int8, device=DEV),
            signs_i8=torch.zeros((mw, R, C), dtype=torch.int8, device=DEV) if int8 else None))
    return mats


# The default shapes run the one-tile-per-block kernels; the "walk" set
# (bf16, packed signs, k loop of at least 12 slices) runs the final product's
# persistent tile walk, wide and tall, with several tiles per workgroup; the
# "units" set has 128 (matrix, worker) units, so that spectral scaling runs
# its power iteration in one launch.
SHAPES = {"default": ([(256, 640), (640, 256), (100, 130)], 4),
          "walk": ([(384, 1024), (1024, 384), (768, 3072)], 8),
          "units": ([(256, 512), (512, 256)] * 8, 8)}


@pytest.mark.parametrize("payload,k,shapes,norm",
                         [(p, k, "default", "frobenius") for p in ("bits", "int8") for k in (0, 1, 3)]
                         + [("bits", 1, "walk", "frobenius"), ("bits", 2, "walk", "frobenius"),
                            ("bits", 1, "walk", "spectral"), ("int8", 2, "default", "spectral"),
                            ("bits", 1, "units", "spectral")])
def test_captured_step_replays_like_eager_steps(payload, k, shapes, norm):
    shapes, mw = SHAPES[shapes]
    int8 = payload == "int8"
    spectral = norm == "spectral"
    p = sm.Params(workers=mw, beta=0.9, eta=1e-3, ns_iters=k, mom_dtype=sm.BF16, ns_dtype=sm.BF16,
                  payload=sm.PAYLOAD_INT8 if int8 else sm.PAYLOAD_BITS,
                  norm=sm.NORM_SPECTRAL if spectral else sm.NORM_FROBENIUS, power_iters=6 if spectral else 0)
    graphed, eager = state(shapes, mw, 50, int8), state(shapes, mw, 50, int8)
    ws_g, ws_e = sm.workspace_tensor(graphed, p, DEV), sm.workspace_tensor(eager, p, DEV)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            sm.signmuon_step(graphed, p, ws_g)  # recorded, not run
    torch.cuda.synchronize()
    for t in range(3):
        g.replay()
        sm.signmuon_step(eager, p, ws_e)
        torch.cuda.synchronize()
        for j, (a, b) in enumerate(zip(graphed, eager)):
            np.testing.assert_array_equal(to_host(a.momentum), to_host(b.momentum), err_msg=f"M {j} t {t}")
            if int8:
                np.testing.assert_array_equal(to_host(a.signs_i8), to_host(b.signs_i8))
            else:
                np.testing.assert_array_equal(to_host(a.packed), to_host(b.packed))
            np.testing.assert_array_equal(to_host(a.vote_out), to_host(b.vote_out))
            np.testing.assert_array_equal(to_host(a.weight), to_host(b.weight), err_msg=f"W {j} t {t}")
        # eager work of the program between replays
        for a in graphed:
            a.grad.mul_(1.0)
        torch.cuda.synchronize()


@pytest.mark.parametrize("payload", ["bits", "int8"])
def test_prepared_calls_equal_plain_calls(payload):
    """sm.Prepared (buffers checked and marshalled once) gives the plain
    calls' results bit for bit over two steps, with new gradients copied into
    the same buffers between them."""
    shapes, mw = [(256, 640), (640, 256), (100, 130)], 3
    int8 = payload == "int8"
    p = sm.Params(workers=mw, beta=0.9, eta=1e-3, ns_iters=2, mom_dtype=sm.BF16, ns_dtype=sm.BF16,
                  payload=sm.PAYLOAD_INT8 if int8 else sm.PAYLOAD_BITS)
    a, b = state(shapes, mw, 70, int8), state(shapes, mw, 70, int8)
    ws_a, ws_b = sm.workspace_tensor(a, p, DEV), sm.workspace_tensor(b, p, DEV)
    prep = sm.Prepared(a, p, ws_a)
    for t in range(2):
        prep.step()
        sm.signmuon_step(b, p, ws_b)
        torch.cuda.synchronize()
        for x, y in zip(a, b):
            np.testing.assert_array_equal(to_host(x.momentum), to_host(y.momentum))
            np.testing.assert_array_equal(to_host(x.weight), to_host(y.weight))
            np.testing.assert_array_equal(to_host(x.vote_out), to_host(y.vote_out))
        for j, (x, y) in enumerate(zip(a, b)):
            g = torch.from_numpy(np.stack([synthetic.random_matrix(900 + 10 * j + m + t, x.shape, 1e-3)
                                           for m in range(mw)])).to(DEV)
            x.grad.copy_(g)
            y.grad.copy_(g)
