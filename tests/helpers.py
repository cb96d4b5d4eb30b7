"""Shared test utilities: running the oracle on a window, tolerance checks,
and snapshots of GPU state.  Test infrastructure only."""
from __future__ import annotations

import os

import numpy as np

import oracle

# Largest observed err / limit per test and per check (printed by the
# conftest's terminal summary).  "rows_tight" and "v_tight" hold the ratio
# against the bound without the propagated gradient error, which shows how
# much of the allowed error the propagation term is actually needed for.
RATIOS: dict[str, dict[str, float]] = {}


def record_ratio(kind: str, err: np.ndarray, lim: np.ndarray) -> None:
    if err.size == 0:
        return
    with np.errstate(invalid="ignore", divide="ignore"):
        r = np.where(np.isfinite(err), err / lim, np.inf)
    test = os.environ.get("PYTEST_CURRENT_TEST", "?").split(" ")[0]
    d = RATIOS.setdefault(test, {})
    d[kind] = max(d.get(kind, 0.0), float(np.max(r)))


def out_of_bounds(err: np.ndarray, lim: np.ndarray) -> np.ndarray:
    """True where err exceeds lim, and where err is NaN (a NaN on one side
    only); comparisons of non-finite values are made explicitly elsewhere."""
    return ~(err <= lim)


def bf16_ordered(u16: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> integers ordered like the values (for ulp distance)."""
    x = u16.astype(np.int64)
    return np.where(x & 0x8000, -(x & 0x7FFF), x)


def f32_ordered(f: np.ndarray) -> np.ndarray:
    x = np.ascontiguousarray(f, np.float32).view(np.int32).astype(np.int64)
    return np.where(x < 0, -(x & 0x7FFFFFFF), x)


def ulp_bf16(a_u16: np.ndarray, b_u16: np.ndarray) -> np.ndarray:
    return np.abs(bf16_ordered(a_u16) - bf16_ordered(b_u16))


def ulp_f32(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    return np.abs(f32_ordered(a) - f32_ordered(b))


def oracle_rows(w_or_cfg, tok: np.ndarray, rows, seeds=(1, 2)):
    """(row_b, neg_b, row_t, neg_t) of one micro-step from the oracle."""
    vocab = w_or_cfg.vocab
    eos = w_or_cfg.eos_id
    rb, nb, rt, nt, _ = oracle.ngram_rows(tok, vocab, eos, rows, seeds)
    return rb, nb, rt, nt


def oracle_window(vocab: int, eos: int, rows, toks: list, dys: list, seeds=(1, 2),
                  keep_rows=None):
    """Oracle window gradient per channel.  Returns a list of two
    (touched, G, absbound) where absbound[u] = sum over the row's positions of
    |dY| (the scale of the fp32 summation error).  With keep_rows[c] (a set
    of row ids as a sorted array) only entries hashed to those rows are fed
    to the oracle, which leaves those rows' sums exact and skips the rest."""
    out = []
    per_c = [[], []]
    negs = [[], []]
    for tok in toks:
        rb, nb, rt, nt, _ = oracle.ngram_rows(tok, vocab, eos, rows, seeds)
        per_c[0].append(rb); negs[0].append(nb)
        per_c[1].append(rt); negs[1].append(nt)
    dY = np.concatenate(dys) if len(dys) else np.zeros((0, 768), np.float32)
    for c in range(2):
        r = np.concatenate(per_c[c]) if per_c[c] else np.zeros(0, np.int64)
        n = np.concatenate(negs[c]) if negs[c] else np.zeros(0, np.uint8)
        d = dY
        if keep_rows is not None:
            m = np.isin(r, keep_rows[c])
            r, n, d = r[m], n[m], dY[m]
        touched, G = oracle.window_grad(r, n, d)
        _, A = oracle.window_grad(r, np.zeros_like(n), np.abs(d))
        out.append((touched, G, A))
    return out


def assert_grad_close(G_gpu: np.ndarray, G_orc: np.ndarray, absbound: np.ndarray, rel=1e-5):
    """|g - o| <= rel * sum|s dY| (per element) + 1e-30."""
    err = np.abs(G_gpu.astype(np.float64) - G_orc.astype(np.float64))
    lim = rel * absbound.astype(np.float64) + 1e-30
    record_ratio("grad", err, lim)
    bad = out_of_bounds(err, lim)
    assert not bad.any(), (f"{int(bad.sum())} gradient elements out of tolerance; worst "
                           f"err/lim {float((err / lim).max()):.3g}")


def grad_bound(absbound: np.ndarray, rel: float = 1e-5) -> np.ndarray:
    """Allowed per-element error of a window gradient (fp32 summation)."""
    return rel * absbound.astype(np.float64) + 1e-30


def spacing_bf16(x_u16: np.ndarray) -> np.ndarray:
    """Distance from a bf16 value to the next one away from zero."""
    a = (x_u16.astype(np.uint32) & 0x7FFF)
    nxt = np.minimum(a + 1, 0x7F7F)
    lo = (a << 16).view(np.float32).astype(np.float64)
    hi = (nxt << 16).view(np.float32).astype(np.float64)
    return np.where(a >= 0x7F7F, np.inf, hi - lo)


def bf16_values(x_u16: np.ndarray) -> np.ndarray:
    return (x_u16.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def rows_limit(W_gpu, W_orc, W_before, dtype: str, absbound=None, v_orc=None, lr=0.0, eps=1.0):
    """Allowed |W_gpu - W_orc| per element, in value space:
        one ulp of the result (in the table dtype)
      + 1e-5 |update|            (fp32 rounding of sqrt, divide, scale * G)
      + lr * dG / (sqrt(v) + eps) (the window gradient's allowed error dG)
    Where W - update cancels to far below the operands, the middle terms
    dominate: no implementation can resolve that result to one ulp of itself."""
    if dtype == "bf16":
        g, o, b = bf16_values(W_gpu), bf16_values(W_orc), bf16_values(W_before)
        ulp = np.maximum(spacing_bf16(W_gpu), spacing_bf16(W_orc))
    else:
        g, o, b = (np.asarray(x, np.float64) for x in (W_gpu, W_orc, W_before))
        ulp = np.maximum(np.spacing(np.abs(np.asarray(W_gpu, np.float32))),
                         np.spacing(np.abs(np.asarray(W_orc, np.float32)))).astype(np.float64)
    lim = ulp + 1e-5 * np.abs(o - b)
    record_ratio("rows_tight", np.abs(g - o), lim)
    if absbound is not None:
        den = np.sqrt(v_orc.astype(np.float64)) + float(np.float32(eps))
        lim = lim + float(np.float32(lr)) * grad_bound(absbound) / den[:, None]
    return np.abs(g - o), lim


def assert_rows_close(W_gpu, W_orc, W_before, dtype: str, G=None, absbound=None, v_orc=None,
                      lr=0.0, eps=1.0):
    err, lim = rows_limit(W_gpu, W_orc, W_before, dtype, absbound, v_orc, lr, eps)
    record_ratio("rows", err, lim)
    bad = out_of_bounds(err, lim)
    assert not bad.any(), (f"{int(bad.sum())} {dtype} table values out of tolerance; worst "
                           f"err/lim {float((err / lim).max()):.3g}")


def assert_v_close(v_gpu, v_orc, rel=1e-5, G=None, absbound=None, beta2=0.0):
    """|g - o| <= 1e-5 |o| plus, when the gradient is given, the change of
    (1 - beta2) mean(G^2) its allowed error can cause."""
    err = np.abs(v_gpu.astype(np.float64) - v_orc.astype(np.float64))
    lim = rel * np.abs(v_orc.astype(np.float64)) + 1e-38
    record_ratio("v_tight", err, lim)
    if absbound is not None:
        d = grad_bound(absbound)
        g = np.abs(G.astype(np.float64))
        lim = lim + (1.0 - float(np.float32(beta2))) * np.mean(2 * g * d + d * d, axis=1)
    record_ratio("v", err, lim)
    bad = out_of_bounds(err, lim)
    assert not bad.any(), f"v out of tolerance: worst err/lim {float((err / lim).max()):.3g}"
