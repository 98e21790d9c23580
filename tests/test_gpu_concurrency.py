"""The library keeps no state between calls: two host threads, each driving its
own stream with its own matrices and workspace, run whole steps at the same time,
and every result equals that of the same steps run one after the other on one
stream. The shapes cover the one-tile-per-block product, the persistent walk of
the final product (wide and tall) and the split-k Gram with its reduce."""
import threading

import numpy as np
import pytest
import torch

import sign_muon_step_amd as sm
import synthetic
from gpu_util import DEV, announce, to_dev, to_host

pytestmark = pytest.mark.gpu

SHAPES = [(384, 1024), (1024, 384), (256, 640), (64, 2304), (100, 130)]
MW = 4


@pytest.fixture(autouse=True)
def _name_the_case(request):
    announce(f"[gpu-test] {request.node.nodeid}")
    yield
    torch.cuda.synchronize()


def state(seed, int8):
    mats = []
    for j, (R, C) in enumerate(SHAPES):
        g = np.stack([synthetic.random_matrix(seed + 10 * j + m, (R, C), 1e-3) for m in range(MW)])
        mats.append(sm.Matrix(
            grad=to_dev(g), momentum=torch.zeros((MW, R, C), dtype=torch.bfloat16, device=DEV),
            packed=None if int8 else torch.zeros((MW, sm.signmuon_packed_words(R * C)),
                                                 dtype=torch.int64, device=DEV),
            weight=to_dev(synthetic.random_matrix(seed + 10 * j + 9, (R, C), 0.02)),
            vote_out=torch.zeros((R, C), dtype=torch.int8, device=DEV),
            signs_i8=torch.zeros((MW, R, C), dtype=torch.int8, device=DEV) if int8 else None))
    return mats


def assert_same(a, b, int8, what):
    for j, (x, y) in enumerate(zip(a, b)):
        np.testing.assert_array_equal(to_host(x.momentum), to_host(y.momentum), err_msg=f"{what} M {j}")
        if int8:
            np.testing.assert_array_equal(to_host(x.signs_i8), to_host(y.signs_i8), err_msg=f"{what} S {j}")
        else:
            np.testing.assert_array_equal(to_host(x.packed), to_host(y.packed), err_msg=f"{what} P {j}")
        np.testing.assert_array_equal(to_host(x.vote_out), to_host(y.vote_out), err_msg=f"{what} V {j}")
        np.testing.assert_array_equal(to_host(x.weight), to_host(y.weight), err_msg=f"{what} W {j}")


@pytest.mark.parametrize("payload,k", [("bits", 1), ("bits", 2), ("int8", 1)])
def test_two_threads_on_two_streams_match_serial_steps(payload, k):
    int8 = payload == "int8"
    p = sm.Params(workers=MW, beta=0.9, eta=1e-3, ns_iters=k, mom_dtype=sm.BF16, ns_dtype=sm.BF16,
                  payload=sm.PAYLOAD_INT8 if int8 else sm.PAYLOAD_BITS)
    seeds = (310, 520)
    concurrent = [state(s, int8) for s in seeds]
    serial = [state(s, int8) for s in seeds]
    ws_c = [sm.workspace_tensor(m, p, DEV) for m in concurrent]
    ws_s = [sm.workspace_tensor(m, p, DEV) for m in serial]
    streams = [torch.cuda.Stream() for _ in seeds]
    torch.cuda.synchronize()

    errors = []

    def run(i):
        try:
            with torch.cuda.stream(streams[i]):
                for _ in range(3):
                    sm.signmuon_step(concurrent[i], p, ws_c[i])
            streams[i].synchronize()
        except Exception as e:  # reported in the main thread
            errors.append(e)

    threads = [threading.Thread(target=run, args=(i,)) for i in range(len(seeds))]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    assert not errors, errors

    for i in range(len(seeds)):
        for _ in range(3):
            sm.signmuon_step(serial[i], p, ws_s[i])
    torch.cuda.synchronize()
    for i in range(len(seeds)):
        assert_same(concurrent[i], serial[i], int8, f"state {i}")
