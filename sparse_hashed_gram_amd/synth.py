"""Seeded synthetic inputs shared by the HIP path's tests, the oracle's tests
and the benchmark.

Nothing here computes any part of the n-gram method (no context, hashing,
gathering, reduction or optimizer arithmetic).  It only draws token ids,
document boundaries, upstream gradients and initial table values.

Recipe (numpy PCG64, seeds ``SeedSequence([workload id, stream, step])``):

* token ids: Zipf(s) over ranks 1..V by inverse CDF (fp64 cumulative sum +
  ``searchsorted``), id = rank - 1, so id 0 is the most frequent;
* collision-stress streams: each token is replaced with probability
  ``hot_frac`` by a uniform draw from a hot set (the first ``hot_size`` ids of
  a seeded permutation of the vocabulary without the EoS id);
* documents: ``fixed512`` puts an EoS at every 512th position; ``geometric``
  starts every micro-step with an EoS (batches are aligned to EoS in the
  speedrun, modded-nanogpt README technique list) and draws document lengths
  from Geometric(1/doc_mean) clipped to [2, doc_max], placing an EoS at each
  document start;
* upstream gradients dY: N(0, 1) float32;
* initial table values: N(0, 0.02).
"""
from __future__ import annotations

import numpy as np

from .workloads import Workload

STREAM_TOKENS = 0
STREAM_DOCLEN = 1
STREAM_DY = 2
STREAM_INIT = 3
STREAM_HOT = 4


def rng(wid: int, stream: int, step: int = 0) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([wid, stream, step])))


_cdf_cache: dict[tuple[int, float], np.ndarray] = {}


def zipf_cdf(vocab: int, s: float) -> np.ndarray:
    key = (vocab, s)
    if key not in _cdf_cache:
        ranks = np.arange(1, vocab + 1, dtype=np.float64)
        p = ranks ** (-s)
        c = np.cumsum(p)
        _cdf_cache[key] = c / c[-1]
    return _cdf_cache[key]


def hot_set(w: Workload) -> np.ndarray:
    r = rng(w.wid, STREAM_HOT, 0)
    ids = np.arange(w.vocab, dtype=np.int64)
    ids = ids[ids != w.eos_id]
    return r.permutation(ids)[: w.hot_size]


def tokens(w: Workload, step: int, T: int | None = None) -> np.ndarray:
    """int32 token ids of one micro-step."""
    T = w.tokens_per_step if T is None else T
    r = rng(w.wid, STREAM_TOKENS, step)
    cdf = zipf_cdf(w.vocab, w.zipf_s)
    u = r.random(T)
    ids = np.searchsorted(cdf, u, side="right").astype(np.int64)
    ids = np.minimum(ids, w.vocab - 1)
    if w.hot_frac > 0:
        hs = hot_set(w)
        pick = r.random(T) < w.hot_frac
        ids[pick] = hs[r.integers(0, len(hs), size=int(pick.sum()))]
    if T == 0:
        return ids.astype(np.int32)
    if w.doc_layout == "fixed512":
        ids[::512] = w.eos_id
    else:
        rd = rng(w.wid, STREAM_DOCLEN, step)
        pos = 0
        while pos < T:
            ids[pos] = w.eos_id
            L = int(rd.geometric(1.0 / w.doc_mean))
            pos += min(max(L, 2), w.doc_max)
    return ids.astype(np.int32)


def dY(w: Workload, step: int, T: int | None = None) -> np.ndarray:
    """float32 [T, dim] upstream gradient of one micro-step."""
    T = w.tokens_per_step if T is None else T
    r = rng(w.wid, STREAM_DY, step)
    return r.standard_normal((T, w.dim), dtype=np.float32)


def init_rows(w: Workload, channel: int, n_rows: int) -> np.ndarray:
    """float32 [n_rows, dim] initial values N(0, 0.02) (host-side tables)."""
    r = rng(w.wid, STREAM_INIT, channel)
    return (r.standard_normal((n_rows, w.dim), dtype=np.float32) * np.float32(0.02))


def doc_starts(tok: np.ndarray, eos_id: int) -> np.ndarray:
    return np.flatnonzero(tok == eos_id)


# ------------------------------------------------------- sampled softmax

STREAM_SSM_X = 5
STREAM_SSM_W = 6
STREAM_SSM_PERM = 7
STREAM_SSM_G = 8
SSM_WID = 100   # seed-space id of the sampled-softmax inputs


def ssm_inputs(step: int, T: int, V: int, w: Workload | None = None):
    """Inputs of one sampled-softmax batch, as float32 arrays holding values
    the caller rounds to bf16 once (X, W) before both sides see them.

    targets: the next tokens of a Zipf stream (``tokens`` of workload w, the
    full-table stream by default, shifted by one); X: final hidden states,
    N(0, 1); W: the lm_head, N(0, 0.05) (logits of standard deviation about
    1.4 at dim 768); perm: a uniform random permutation of [0, V), the
    randomness the candidate draw uses; g: per-position upstream gradients,
    uniform in [0.5, 1.5) / T."""
    from .workloads import FULL
    w = w or FULL
    tgt = tokens(w, step, T + 1)[1:].astype(np.int32) % V
    X = rng(SSM_WID, STREAM_SSM_X, step).standard_normal((T, 768), dtype=np.float32)
    W = rng(SSM_WID, STREAM_SSM_W, 0).standard_normal((V, 768), dtype=np.float32) * np.float32(0.05)
    perm = rng(SSM_WID, STREAM_SSM_PERM, step).permutation(V).astype(np.int32)
    g = (rng(SSM_WID, STREAM_SSM_G, step).random(T) + 0.5).astype(np.float32) / np.float32(max(T, 1))
    return tgt, X, W, perm, g
