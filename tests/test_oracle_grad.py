"""Pins of the oracle's window gradient and touched-row set (CPU only).

The backward of the signed gather is the transpose product S^T dY, summed
over the micro-steps of one update window (updates every 4 steps on the
accumulated gradient: @classiclarryd post quoted on the airebao.com item;
modded-nanogpt README technique list).  numpy's dense fp64 matmul is the
independent route; the touched set must be exactly the distinct rows.
"""
import numpy as np

import oracle
from oracle import dense
from sparse_hashed_gram_amd import synth, workloads


def _window(w, first_step, R, n_steps=4, T=None):
    rows_b, neg_b, rows_t, neg_t, dys, toks = [], [], [], [], [], []
    for s in range(first_step, first_step + n_steps):
        tok = synth.tokens(w, s, T)
        rb, nb, rt, nt, _ = oracle.ngram_rows(tok, w.vocab, w.eos_id, R)
        rows_b.append(rb); neg_b.append(nb); rows_t.append(rt); neg_t.append(nt)
        dys.append(synth.dY(w, s, T)); toks.append(tok)
    cat = np.concatenate
    return cat(rows_b), cat(neg_b), cat(rows_t), cat(neg_t), cat(dys), toks


def _ulp_diff(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    ia = a.view(np.int32).astype(np.int64)
    ib = b.view(np.int32).astype(np.int64)
    ia = np.where(ia < 0, -(ia & 0x7FFFFFFF), ia)
    ib = np.where(ib < 0, -(ib & 0x7FFFFFFF), ib)
    return np.abs(ia - ib)


def test_window_grad_equals_transpose_product():
    w = workloads.TINY
    R = w.rows
    rb, nb, rt, nt, dY, _ = _window(w, 0, R, T=1024)
    for rows, neg, Rc in ((rb, nb, R[0]), (rt, nt, R[1])):
        touched, G = oracle.window_grad(rows, neg, dY)
        np.testing.assert_array_equal(touched, np.unique(rows))
        ref = dense.grad(dense.selection_matrix(rows, neg, Rc), dY)
        ref32 = ref[touched].astype(np.float32)
        assert _ulp_diff(G, ref32).max() <= 1
        # rows never touched get nothing
        untouched = np.setdiff1d(np.arange(Rc), touched)
        assert np.all(ref[untouched] == 0)


def test_adjoint_identity():
    # <S_b W_b + S_t W_t, dY> == <W_b, S_b^T dY> + <W_t, S_t^T dY>
    w = workloads.TINY
    R = (512, 700)
    rs = np.random.default_rng(7)
    Wb = (rs.standard_normal((R[0], 768)) * 0.02).astype(np.float32)
    Wt = (rs.standard_normal((R[1], 768)) * 0.02).astype(np.float32)
    tok = synth.tokens(w, 3)
    dY = synth.dY(w, 3)
    rb, nb, rt, nt, _ = oracle.ngram_rows(tok, w.vocab, w.eos_id, R)
    out = oracle.forward(Wb, Wt, rb, nb, rt, nt).astype(np.float64)
    lhs = float((out * dY.astype(np.float64)).sum())
    ub, Gb = oracle.window_grad(rb, nb, dY)
    ut, Gt = oracle.window_grad(rt, nt, dY)
    rhs = float((Wb[ub].astype(np.float64) * Gb).sum() + (Wt[ut].astype(np.float64) * Gt).sum())
    assert abs(lhs - rhs) <= 1e-5 * (np.abs(out * dY).sum())


def test_opposite_signs_cancel_exactly():
    # R = 1: every n-gram shares row 0.  Two positions with opposite signs and
    # equal upstream gradients contribute nothing.
    w = workloads.TINY
    tok = synth.tokens(w, 4)[:64]
    rb, nb, *_ = oracle.ngram_rows(tok, w.vocab, w.eos_id, (1, 1))
    i = int(np.flatnonzero(nb == 0)[0])
    j = int(np.flatnonzero(nb == 1)[0])
    dY = np.zeros((len(tok), 768), np.float32)
    dY[i] = dY[j] = np.linspace(-3, 3, 768, dtype=np.float32)
    touched, G = oracle.window_grad(rb, nb, dY)
    assert touched.tolist() == [0]
    assert np.all(G == 0)


def test_single_token_gradient_is_signed_dy():
    dY = np.random.default_rng(5).standard_normal((1, 768)).astype(np.float32)
    for neg in (0, 1):
        touched, G = oracle.window_grad(np.array([42]), np.array([neg], np.uint8), dY)
        assert touched.tolist() == [42]
        np.testing.assert_array_equal(G[0], -dY[0] if neg else dY[0])


def test_empty_window():
    touched, G = oracle.window_grad(np.zeros(0, np.int64), np.zeros(0, np.uint8),
                                    np.zeros((0, 768), np.float32))
    assert len(touched) == 0 and G.shape == (0, 768)
