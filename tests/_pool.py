"""Process pool that runs the CPU oracle on pieces of the full-size workloads.

Test infrastructure: the GPU tests hand the oracle whole benchmark-sized
inputs (every calibration token, every expert), which one Python process
would take minutes over.  The oracle's definitions are independent per
channel group, per weight row and per expert, so the pieces below run in a
pool of spawned worker processes (no GPU state is inherited; each worker
imports numpy and the oracle only, with one BLAS thread).  Nothing here
holds method arithmetic: every function calls the oracle on its piece.
"""
from __future__ import annotations

import concurrent.futures as cf
import multiprocessing as mp
import os

import numpy as np


def n_workers() -> int:
    # at most 16: the host share of one GPU on the test machines
    return max(1, min(16, len(os.sched_getaffinity(0))))


def _init() -> None:
    try:
        from threadpoolctl import threadpool_limits
        threadpool_limits(1)
    except Exception:
        pass


def make_pool() -> cf.ProcessPoolExecutor:
    return cf.ProcessPoolExecutor(max_workers=n_workers(), mp_context=mp.get_context("spawn"),
                                  initializer=_init)


# ---------------------------------------------------------------- work items

def hessian_piece(x_bits: np.ndarray):
    """(H of the piece's groups in float64, amax of the piece)."""
    from oracle import nvfp4 as N
    return N.hessian(x_bits), N.tensor_scale(x_bits)[0]


def sweep_costs_piece(w_bits: np.ndarray, h: np.ndarray, s2: float) -> np.ndarray:
    """Cost of every code for every block of the rows in w_bits: [rows, G, 127]."""
    from oracle import nvfp4 as N
    return N.sweep_costs(w_bits, h, s2)


def cast_piece(packed: np.ndarray, e8m0: np.ndarray):
    """The oracle's cast of a slice of groups (experts)."""
    from oracle import mxcast as M
    return M.mxfp4_to_nvfp4(packed, e8m0)


# ---------------------------------------------------------------- drivers

def sweep_costs(pool, w_bits: np.ndarray, h: np.ndarray, s2: float, rows_per_item: int = 16) -> np.ndarray:
    """sweep_costs over row tiles in the pool, concatenated in row order."""
    futs = [pool.submit(sweep_costs_piece, np.ascontiguousarray(w_bits[r:r + rows_per_item]), h, s2)
            for r in range(0, w_bits.shape[0], rows_per_item)]
    return np.concatenate([f.result() for f in futs], axis=0)


def cast(pool, packed: np.ndarray, e8m0: np.ndarray):
    """The oracle's cast, one expert per work item; outputs stacked by expert."""
    futs = [pool.submit(cast_piece, np.ascontiguousarray(packed[g:g + 1]), np.ascontiguousarray(e8m0[g:g + 1]))
            for g in range(packed.shape[0])]
    res = [f.result() for f in futs]
    return tuple(np.concatenate([r[i] for r in res], axis=0) for i in range(4))
