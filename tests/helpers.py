"""Shared test utilities: running the oracle on a window, tolerance checks,
and snapshots of GPU state.  Test infrastructure only."""
from __future__ import annotations

import numpy as np

import oracle


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
    bad = err > lim
    assert not bad.any(), (f"{int(bad.sum())} gradient elements out of tolerance; worst "
                           f"err/lim {float((err / lim).max()):.3g}")


def assert_rows_close(W_gpu, W_orc, W_before, dtype: str):
    """bf16: <= 1 ulp.  fp32: |g - o| <= 1e-5 |update| + 1 ulp."""
    if dtype == "bf16":
        d = ulp_bf16(W_gpu, W_orc)
        assert d.max(initial=0) <= 1, f"bf16 rows differ by up to {int(d.max())} ulp"
    else:
        upd = np.abs(W_orc.astype(np.float64) - W_before.astype(np.float64))
        err = np.abs(W_gpu.astype(np.float64) - W_orc.astype(np.float64))
        ulp = np.spacing(np.abs(W_orc)).astype(np.float64)
        bad = err > 1e-5 * upd + ulp
        assert not bad.any(), f"{int(bad.sum())} fp32 table values out of tolerance"


def assert_v_close(v_gpu, v_orc, rel=1e-5):
    err = np.abs(v_gpu.astype(np.float64) - v_orc.astype(np.float64))
    assert np.all(err <= rel * np.abs(v_orc.astype(np.float64)) + 1e-38), \
        f"v out of tolerance: worst rel {float((err / (np.abs(v_orc) + 1e-38)).max()):.3g}"
