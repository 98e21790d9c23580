#!/usr/bin/env python3
"""Writes the stored oracle results of the large transformer-block workload
(4 x 4096x4096, 4096x11008, 11008x4096; 16 workers, bf16 momentum and
Newton-Schulz, 5 iterations) that the GPU test compares against.

The oracle takes minutes to an hour per matrix at these sizes, too long to
run inside a GPU test, so this script runs it once, offline, for worker 0 of
each distinct shape at step 0 (momentum from zero). It calls only the CPU
oracle (``oracle/``) and the seeded input generators (``synthetic/``).

Each ``block4096_k5_m<j>_w<w>.npz`` holds, for matrix j and worker w:
  mom_sha256  sha256 of the stored bf16 momentum (the oracle's O1): the GPU
              test checks that its own momentum hashes the same, so both
              sides start from identical inputs;
  sign_rows   the rows whose packed signs are stored (every row of the
              4096x4096 matrix, a seeded band of rows of the others);
  signs       those rows' signs, 1 bit per entry, LSB first (numpy
              packbits, bitorder little), row by row;
  near_zero   flat indices (within sign_rows' entries) of |U| < 1e-6 max|U|,
              where either sign is correct within rounding;
  u_rows / u  a seeded set of whole rows of U and their fp32 values;
  fro, max_abs  ||U||_F and max|U| of the whole matrix (fp64).

Usage: python tests/golden/make_block4096_golden.py [j ...]   (default 0 4 5)
Run from the repository root; cases run in parallel processes.
"""
import hashlib
import os
import sys
import time
from concurrent.futures import ProcessPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

import oracle  # noqa: E402
import synthetic  # noqa: E402

WORKLOAD = "block4096_mw16_k5"
# (matrix index, worker, rows whose signs are stored, whole U rows stored)
CASES = {0: (0, 4096, 256), 4: (0, 1024, 64), 5: (0, 1024, 128)}


def path_for(j: int, w: int) -> str:
    return os.path.join(HERE, f"block4096_k5_m{j}_w{w}.npz")


def make(j: int) -> str:
    wl = synthetic.WORKLOADS[WORKLOAD]
    w, n_sign_rows, n_u_rows = CASES[j]
    R, C = wl.shapes[j]
    t0 = time.time()
    g = synthetic.gradient(wl, j, w, 0)
    m = np.zeros((R, C), np.uint16)          # bf16 momentum, M_0 = 0
    oracle.momentum(g, m, wl.beta)
    _, x0 = oracle.normalise(m)
    u = oracle.newton_schulz(x0, wl.ns_iters, oracle.BF16)
    rng = np.random.default_rng(20260519 + j)
    if n_sign_rows >= R:
        sign_rows = np.arange(R, dtype=np.int64)
    else:
        start = int(rng.integers(0, R - n_sign_rows + 1))
        sign_rows = np.arange(start, start + n_sign_rows, dtype=np.int64)
    band = u[sign_rows]
    max_abs = float(np.abs(u).max())
    signs = np.packbits((band >= 0).astype(np.uint8), axis=1, bitorder="little")
    near_zero = np.flatnonzero(np.abs(band) < 1e-6 * max_abs).astype(np.int64)
    u_rows = np.sort(rng.choice(R, n_u_rows, replace=False)).astype(np.int64)
    np.savez_compressed(
        path_for(j, w), workload=WORKLOAD, matrix=j, worker=w, step=0, ns_iters=wl.ns_iters,
        shape=np.array([R, C], np.int64),
        mom_sha256=hashlib.sha256(m.tobytes()).hexdigest(),
        sign_rows=sign_rows, signs=signs, near_zero=near_zero, u_rows=u_rows,
        u=u[u_rows].astype(np.float32), fro=float(np.linalg.norm(u)), max_abs=max_abs)
    return f"matrix {j} {R}x{C} worker {w}: {time.time() - t0:.0f} s -> {path_for(j, w)}"


def main():
    js = [int(a) for a in sys.argv[1:]] or sorted(CASES)
    with ProcessPoolExecutor(max_workers=len(js)) as ex:
        for msg in ex.map(make, js):
            print(msg, flush=True)


if __name__ == "__main__":
    main()
