"""CPU oracle of the sampled-softmax training loss (numpy, fp64).

TEST INFRASTRUCTURE, like the rest of ``oracle/``: only ``tests/``,
``__graft_entry__.smoke()`` and ``bench.py``'s CPU-baseline leg use it, and it
shares no code with the HIP library.

What the pages fix: the loss scores only a subset of the vocabulary for most
of training; a vocabulary entry that does not occur in the batch has its
lm_head forward and backward skipped some of the time (the @classiclarryd post
quoted on the airebao.com item); the candidate set is shared and its size
follows a schedule of 10,240, 14,336 and 24,576 entries, then all 50,304 for
the last steps (agentic-affairs.com, "NanoGPT Training Record", Key
Optimizations and Ablation Table Results, sampled-softmax item; Technical
Architecture and Implementation Details).

Readings where the pages are silent, taken identically by the HIP path:

- candidate set S of exactly C ids: every id that occurs among the batch's
  targets, in ascending order, then ids that do not occur, in the order of a
  caller-supplied random permutation of the vocabulary, until |S| = C.  An id
  absent from the batch is thus scored with probability (C - n) / (V - n).
  If the batch holds more than C distinct targets the call is invalid
  (``candidates`` reports it; the HIP path flags it and voids the call);
- logits z = X W_S^T with no bias, scale or cap; the loss of a position is
  the cross-entropy over S only: log sum_{c in S} exp(z_c) - z_{target}, with
  no correction for the sampling;
- the backward takes a per-position upstream gradient g (1/T for a mean):
  dz = g (softmax_S(z) - onehot(target)), dX = dz W_S, dW[S[c]] += (dz^T X)[c];
  rows of W outside S receive nothing.

X and W are taken as the values they hold (bf16 inputs are exact in fp64);
every sum is fp64.
"""
from __future__ import annotations

import numpy as np


def candidates(targets: np.ndarray, perm: np.ndarray, V: int, C: int):
    """Candidate set of one batch.

    Returns (cand [C] int64, slot [T] int64, n_present, ok): cand[slot[i]] is
    targets[i].  ok is False when the batch holds more than C distinct
    targets (cand and slot are then None)."""
    targets = np.asarray(targets, np.int64)
    perm = np.asarray(perm, np.int64)
    present = np.zeros(V, bool)
    present[targets] = True
    ids = np.flatnonzero(present)                   # ascending
    n = len(ids)
    if n > C:
        return None, None, n, False
    absent_in_order = perm[~present[perm]]          # permutation order
    cand = np.concatenate([ids, absent_in_order[:C - n]]).astype(np.int64)
    slot = np.searchsorted(ids, targets).astype(np.int64)
    return cand, slot, n, True


def logits(X: np.ndarray, W: np.ndarray, cand: np.ndarray) -> np.ndarray:
    """z[i, c] = X[i] . W[cand[c]] in fp64 ([T, C])."""
    return np.asarray(X, np.float64) @ np.asarray(W, np.float64)[cand].T


def _lse(z: np.ndarray) -> np.ndarray:
    m = z.max(axis=1)
    return m + np.log(np.exp(z - m[:, None]).sum(axis=1))


def loss_fwd(X, W, cand, slot, chunk: int = 4096):
    """(loss [T], lse [T]) in fp64, over the candidate set only.  Positions
    are processed in chunks (each position's loss depends on its own row)."""
    T = len(X)
    loss = np.empty(T, np.float64)
    lse = np.empty(T, np.float64)
    Wc = np.asarray(W, np.float64)[cand]
    slot = np.asarray(slot, np.int64)
    for a in range(0, T, chunk):
        b = min(T, a + chunk)
        z = np.asarray(X[a:b], np.float64) @ Wc.T
        lse[a:b] = _lse(z)
        loss[a:b] = lse[a:b] - z[np.arange(b - a), slot[a:b]]
    return loss, lse


def dlogits(X, W, cand, slot, dloss, lse=None):
    """dz = g (softmax_S(z) - onehot(slot)) in fp64 ([T, C])."""
    z = logits(X, W, cand)
    if lse is None:
        lse = _lse(z)
    p = np.exp(z - np.asarray(lse, np.float64)[:, None])
    p[np.arange(len(z)), np.asarray(slot, np.int64)] -= 1.0
    return np.asarray(dloss, np.float64)[:, None] * p


def loss_bwd(X, W, cand, slot, dloss):
    """(dX [T, D], dWc [C, D]) in fp64: dWc[c] is what row cand[c] of W
    receives; rows outside the candidate set receive nothing."""
    dz = dlogits(X, W, cand, slot, dloss)
    Wc = np.asarray(W, np.float64)[cand]
    return dz @ Wc, dz.T @ np.asarray(X, np.float64)


def dW_rows(X, W, cand, slot, dloss, lse, cs):
    """Rows cs of dWc (what W[cand[cs]] receives), from every position's lse:
    dWc[c] = sum_i g_i (exp(z_ic - lse_i) - [slot_i = c]) X_i, fp64."""
    cs = np.asarray(cs, np.int64)
    X64 = np.asarray(X, np.float64)
    z = X64 @ np.asarray(W, np.float64)[np.asarray(cand)[cs]].T          # [T, |cs|]
    p = np.exp(z - np.asarray(lse, np.float64)[:, None])
    p -= (np.asarray(slot, np.int64)[:, None] == cs[None, :])
    return (np.asarray(dloss, np.float64)[:, None] * p).T @ X64
