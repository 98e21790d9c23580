"""signmuon_step_noalloc: the whole step with the workspace in the library's
static device scratch, for callers that cannot allocate device memory.

It runs the same launches as signmuon_step on a caller's workspace, so its
output must equal that entry point's bit for bit: momentum, U, packed signs,
vote and W. Two calls in a row share the scratch; the second is smaller and
of another kind, so any dependence on what the first left behind would show.
A step whose workspace exceeds SIGNMUON_STATIC_SCRATCH_BYTES is refused with
SIGNMUON_ESCRATCH before any HIP call (checked on the host, without a GPU)."""
import ctypes

import numpy as np
import pytest
import torch

import sign_muon_step_amd as sm
import synthetic


def _state(shapes, mw, mom_t, seed, polar, dev):
    mats = []
    for j, (R, C) in enumerate(shapes):
        g = np.stack([synthetic.random_matrix(seed + 10 * j + m, (R, C), 1e-3) for m in range(mw)])
        mats.append(sm.Matrix(
            grad=torch.from_numpy(g).to(dev),
            momentum=torch.zeros((mw, R, C), dtype=mom_t, device=dev),
            packed=torch.zeros((mw, sm.signmuon_packed_words(R * C)), dtype=torch.int64, device=dev),
            weight=torch.from_numpy(synthetic.random_matrix(seed + 10 * j + 9, (R, C), 0.02)).to(dev),
            polar_out=torch.zeros((mw, R, C), dtype=torch.float32, device=dev) if polar else None,
            vote_out=torch.zeros((R, C), dtype=torch.int8, device=dev)))
    return mats


def _bits(t):
    return t.view({1: torch.int8, 2: torch.int16, 4: torch.int32, 8: torch.int64}[t.element_size()])


def _same(a, b, what):
    for j, (x, y) in enumerate(zip(a, b)):
        for name in ("momentum", "polar_out", "packed", "vote_out", "weight"):
            tx, ty = getattr(x, name), getattr(y, name)
            if tx is not None:
                assert torch.equal(_bits(tx), _bits(ty)), f"{what}: matrix {j} {name} differs"


@pytest.mark.gpu
def test_noalloc_equals_step_on_two_calls():
    dev = torch.device("cuda:0")
    calls = [
        # one GPT-2 small layer, 8 workers, bf16, k = 1, signs from the walk
        dict(shapes=[(768, 2304), (768, 768), (768, 3072), (3072, 768)], mw=8, mom=torch.bfloat16,
             params=sm.Params(workers=8, ns_iters=1, mom_dtype=sm.BF16, ns_dtype=sm.BF16), polar=False),
        # smaller: fp32, 3 workers, k = 2 (iterate buffers), U stored, ragged shapes
        dict(shapes=[(300, 700), (700, 300), (64, 576)], mw=3, mom=torch.float32,
             params=sm.Params(workers=3, ns_iters=2), polar=True),
    ]
    sizes = []
    for i, c in enumerate(calls):
        a = _state(c["shapes"], c["mw"], c["mom"], 500 + i, c["polar"], dev)
        b = _state(c["shapes"], c["mw"], c["mom"], 500 + i, c["polar"], dev)
        nbytes = sm.signmuon_workspace_bytes(a, c["params"])
        assert 0 < nbytes <= sm.STATIC_SCRATCH_BYTES
        sizes.append(nbytes)
        for _ in range(2):  # two steps: the momentum carries over
            sm.signmuon_step_noalloc(a, c["params"])
            sm.signmuon_step(b, c["params"], sm.workspace_tensor(b, c["params"], dev))
            torch.cuda.synchronize()
            _same(a, b, f"call {i}")
    assert sizes[1] < sizes[0]


def test_noalloc_refuses_a_step_beyond_the_scratch():
    """The GPT-2 small batch (48 matrices, 8 workers) needs about 433 MiB of
    workspace: refused with SIGNMUON_ESCRATCH, before any HIP call (fake,
    never dereferenced device addresses; runs without a GPU)."""
    lib = sm.library()
    wl = synthetic.WORKLOADS["gpt2s_mw8_k1"]
    base = 0x7f0000000000
    arr = (sm._Matrix * len(wl.shapes))(*[
        sm._Matrix(R, C, base, base + 0x100000, None, base + 0x300000, base + 0x400000, None, None)
        for R, C in wl.shapes])
    p = sm._Params(8, 0.9, 1e-3, 1, 0, sm.F32, sm.BF16, sm.BF16, 0, 0, 0)
    need = lib.signmuon_workspace_bytes(arr, len(wl.shapes), ctypes.byref(p))
    assert need > sm.STATIC_SCRATCH_BYTES
    rc = lib.signmuon_step_noalloc(arr, len(wl.shapes), ctypes.byref(p), None)
    assert rc == -7
    assert "static scratch" in sm.signmuon_strerror(rc)
