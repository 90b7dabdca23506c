"""Reference of the SO(4) calibration (CPU, NumPy, float64).

TEST INFRASTRUCTURE -- see the package docstring.

The idea card, Implementation notes: start from fixed random SO(4) rotations and
calibrate them on representative vectors by minimising the reconstruction MSE after
3-bit quantisation, each SO(4) block parameterised by a normalised quaternion pair
(R x = a x conj(b) for unit quaternions a, b).

READING (the optimiser is not given): coordinate search.  The objective is the summed
squared reconstruction error of y = B (H x) over the calibration vectors; it splits
over quantisation blocks, so changing block i of B changes only the quantisation
block that holds its four dims.  In sweep s, for i = 0 .. d/4 - 1 in order, every
candidate P_c (c = 0 .. C-1, P_0 = I; the candidates are inputs) gives R_i' = P_c R_i,
and R_i takes the candidate with the smallest error of that quantisation block (the
first one on ties, so the error never increases).  The symmetric quantiser is the
idea card's, in exact arithmetic: s = (max |y| + eps) / L, L = 2^(b-1) - 1, codes
clip(round(y / s), -L, L), error sum (y - s c)^2.
"""
from __future__ import annotations

import numpy as np

from .okv_ref import hadamard

__all__ = ["quat_mul", "quat_rotation", "so4_block_errors", "so4_total_error", "calibrate_so4"]


def quat_mul(p, q) -> np.ndarray:
    """Hamilton product p q of quaternions (w, x, y, z)."""
    p0, p1, p2, p3 = np.asarray(p, dtype=np.float64)
    q0, q1, q2, q3 = np.asarray(q, dtype=np.float64)
    return np.array([p0 * q0 - p1 * q1 - p2 * q2 - p3 * q3,
                     p0 * q1 + p1 * q0 + p2 * q3 - p3 * q2,
                     p0 * q2 - p1 * q3 + p2 * q0 + p3 * q1,
                     p0 * q3 + p1 * q2 - p2 * q1 + p3 * q0])


def quat_rotation(a, b) -> np.ndarray:
    """The 4x4 matrix of x -> a x conj(b) for unit quaternions a, b (columns: images
    of the basis quaternions 1, i, j, k)."""
    a = np.asarray(a, dtype=np.float64) / np.linalg.norm(a)
    b = np.asarray(b, dtype=np.float64) / np.linalg.norm(b)
    bc = b * np.array([1.0, -1.0, -1.0, -1.0])
    return np.stack([quat_mul(quat_mul(a, e), bc) for e in np.eye(4)], axis=1)


def _hx(x):
    x = np.asarray(x, dtype=np.float64)
    return x @ hadamard(x.shape[-1]).T


def _block_error(hx, rot, block: int, blk: int, eps: float, bits: int, override=None) -> float:
    """Squared error of quantisation block `blk` over all vectors, y = B (H x) on the
    block's dims; `override` = (group, matrix) replaces that group's rotation."""
    lev = 2 ** (bits - 1) - 1
    cols = []
    for g in range(blk * block // 4, (blk + 1) * block // 4):
        r = override[1] if override is not None and override[0] == g else rot[g]
        cols.append(hx[:, 4 * g:4 * g + 4] @ np.asarray(r).T)
    y = np.concatenate(cols, axis=1)
    s = (np.abs(y).max(axis=1) + eps) / lev
    safe = np.where(s > 0, s, 1.0)
    c = np.clip(np.round(y / safe[:, None]), -lev, lev)      # numpy rounds half to even
    c = np.where(s[:, None] > 0, c, 0.0)
    return float(np.sum((y - s[:, None] * c) ** 2))


def so4_block_errors(x, rot, block: int, eps: float, bits: int = 3) -> np.ndarray:
    """Per quantisation block: the summed squared reconstruction error of y = B (H x)
    over the vectors x (N, d).  rot: (d/4, 4, 4) rows of B's blocks."""
    hx = _hx(x)
    d = hx.shape[1]
    return np.array([_block_error(hx, rot, block, b, eps, bits) for b in range(d // block)])


def so4_total_error(x, rot, block: int, eps: float, bits: int = 3) -> float:
    return float(so4_block_errors(x, rot, block, eps, bits).sum())


def calibrate_so4(x, rot0, cands, block: int, eps: float, bits: int = 3):
    """Coordinate search (module docstring).  x: (N, d); rot0: (d/4, 4, 4); cands:
    (S, d/4, C, 4, 4) with cands[:, :, 0] = I.  Returns (rot, trace, choice): the
    calibrated rotations, the total error before and after each sweep, and the chosen
    candidate index per (sweep, group)."""
    hx = _hx(x)
    rot = np.array(rot0, dtype=np.float64)
    d = hx.shape[1]
    sweeps, _, n_cand = cands.shape[:3]
    tot = lambda: sum(_block_error(hx, rot, block, b, eps, bits) for b in range(d // block))
    trace = [tot()]
    choice = np.zeros((sweeps, d // 4), dtype=np.int64)
    for s in range(sweeps):
        for g in range(d // 4):
            blk = 4 * g // block
            errs = [_block_error(hx, rot, block, blk, eps, bits, (g, cands[s, g, c] @ rot[g]))
                    for c in range(n_cand)]
            best = int(np.argmin(errs))                           # first minimum
            choice[s, g] = best
            rot[g] = cands[s, g, best] @ rot[g]
        trace.append(tot())
    return rot, np.array(trace), choice
