"""Dense brute-force reference for tiny tables (numpy, fp64).

TEST INFRASTRUCTURE, like the rest of ``oracle/``.

This is the method written without any of its sparsity: the hashed lookup is
an explicit +/-1 selection matrix S (one nonzero per position and channel), the
forward is the matrix product S W, the gradient is S^T dY, and the optimizer
(Adam with beta1 = 0 and one second moment per row, modded-nanogpt README,
technique list; the @classiclarryd post quoted on the airebao.com item) runs
on *every* row at every update step, with a zero gradient for rows the window
did not touch.  The lazy oracle must agree with it: applying beta2 to a row
only when it is next touched, raised to the number of steps it missed, is the
same recursion as decaying it every step with zero gradient.
"""
from __future__ import annotations

import numpy as np


def selection_matrix(rows: np.ndarray, neg: np.ndarray, R: int) -> np.ndarray:
    """S[i, rows[i]] = -1 if neg[i] else +1 (fp64, [T, R])."""
    T = len(rows)
    S = np.zeros((T, R), np.float64)
    S[np.arange(T), rows] = np.where(np.asarray(neg) != 0, -1.0, 1.0)
    return S


def forward(Sb: np.ndarray, Wb: np.ndarray, St: np.ndarray, Wt: np.ndarray) -> np.ndarray:
    """S_b W_b + S_t W_t in fp64."""
    return Sb @ np.asarray(Wb, np.float64) + St @ np.asarray(Wt, np.float64)


def grad(S: np.ndarray, dY: np.ndarray) -> np.ndarray:
    """S^T dY in fp64 ([R, dim])."""
    return S.T @ np.asarray(dY, np.float64)


def step_all_rows(W: np.ndarray, v: np.ndarray, G: np.ndarray, lr: float,
                  beta2: float, eps: float):
    """One dense update of every row: v <- beta2 v + (1 - beta2) mean(G^2),
    W <- W - lr G / (sqrt(v) + eps).  W float32 (rounded after the step), v
    fp64 (kept unrounded), G fp64."""
    lr, beta2, eps = (float(np.float32(x)) for x in (lr, beta2, eps))
    v_new = beta2 * v + (1.0 - beta2) * np.mean(G * G, axis=1)
    W_new = (np.asarray(W, np.float64) - lr * G / (np.sqrt(v_new) + eps)[:, None])
    return W_new.astype(np.float32), v_new
