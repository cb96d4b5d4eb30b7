"""Pins of the oracle's lazy sparse row-wise step (CPU only).

The update is Adam with beta1 = 0 and one second-moment float per 768-wide
row, run only on rows the window touched, with beta2 applied retroactively
when a row is next used (@classiclarryd post quoted on the airebao.com item;
modded-nanogpt README technique list).  The central pin: the lazy form equals
the dense form that updates every row at every step with zero gradient on the
untouched ones.  Closed forms pin the constants (mean vs sum, eps placement,
the decay exponent).
"""
import numpy as np
import pytest

import oracle
from oracle import dense
from sparse_hashed_gram_amd import synth, workloads


def _run_lazy_vs_dense(w, R, n_windows, T, lr, beta2, eps, seed):
    rs = np.random.default_rng(seed)
    dim = w.dim
    W_lazy = [(rs.standard_normal((Rc, dim)) * 0.02).astype(np.float32) for Rc in R]
    W_dense = [x.copy() for x in W_lazy]
    v_lazy = [np.zeros(Rc, np.float32) for Rc in R]
    tl_lazy = [np.zeros(Rc, np.int32) for Rc in R]
    v_dense = [np.zeros(Rc, np.float64) for Rc in R]
    for win in range(n_windows):
        t = win + 1
        rows = [[], []]
        negs = [[], []]
        dys = []
        for m in range(w.accum_steps):
            step = win * w.accum_steps + m
            tok = synth.tokens(w, step, T)
            rb, nb, rt, nt, _ = oracle.ngram_rows(tok, w.vocab, w.eos_id, R)
            rows[0].append(rb); negs[0].append(nb)
            rows[1].append(rt); negs[1].append(nt)
            dys.append(synth.dY(w, step, T))
        dY = np.concatenate(dys)
        for c in range(2):
            rc = np.concatenate(rows[c]); nc = np.concatenate(negs[c])
            touched, G = oracle.window_grad(rc, nc, dY)
            W_lazy_before = W_lazy[c].copy()
            # lazy
            Wn, vn, tn = oracle.sparse_step(G, W_lazy[c][touched], v_lazy[c][touched],
                                            tl_lazy[c][touched], t, lr, beta2, eps)
            W_lazy[c][touched] = Wn
            v_lazy[c][touched] = vn
            tl_lazy[c][touched] = tn
            # dense: every row, zero gradient where untouched
            Gd = dense.grad(dense.selection_matrix(rc, nc, R[c]), dY)
            W_before = W_dense[c].copy()
            W_dense[c], v_dense[c] = dense.step_all_rows(W_dense[c], v_dense[c], Gd,
                                                         lr, beta2, eps)
            untouched = np.setdiff1d(np.arange(R[c]), touched)
            # untouched rows: dense update is exactly zero
            np.testing.assert_array_equal(W_dense[c][untouched], W_before[untouched])
            np.testing.assert_array_equal(W_lazy[c][untouched], W_lazy_before[untouched])
            # touched set and t_last
            assert np.array_equal(np.flatnonzero(tl_lazy[c] == t), touched)
            # v: lazy value decayed to now equals the dense value
            b2 = float(np.float32(beta2))
            v_now = v_lazy[c].astype(np.float64) * b2 ** (t - tl_lazy[c])
            np.testing.assert_allclose(v_now, v_dense[c], rtol=2e-6, atol=0)
            # W: lazy vs dense within 1 ulp of fp32 (v rounding differs)
            upd = np.abs(W_dense[c].astype(np.float64) - W_before.astype(np.float64))
            diff = np.abs(W_lazy[c].astype(np.float64) - W_dense[c].astype(np.float64))
            ulp = np.spacing(np.abs(W_dense[c])).astype(np.float64)
            assert np.all(diff <= 1e-5 * upd + ulp)
            # both forms continue from the same rows, so each window is
            # compared on its own (1-ulp differences do not compound)
            W_dense[c] = W_lazy[c].copy()
    return tl_lazy


def test_lazy_equals_dense_tiny_workload():
    w = workloads.TINY
    _run_lazy_vs_dense(w, w.rows, n_windows=2, T=2048, lr=w.lr, beta2=w.beta2,
                       eps=w.eps, seed=0)


def test_lazy_equals_dense_with_long_gaps():
    # Small T against a larger table: rows go untouched for several windows, so
    # the retroactive beta2^k with k > 1 is exercised.
    w = workloads.TINY
    tl = _run_lazy_vs_dense(w, (2000, 3000), n_windows=10, T=64, lr=0.02, beta2=0.9,
                            eps=1e-6, seed=1)
    gaps = [np.diff(np.sort(np.unique(t))) for t in tl]
    assert any(len(g) for g in gaps)


def test_constant_gradient_closed_form():
    # beta2 = 0, G = c everywhere: mean(G^2) = c^2, v = c^2, sqrt(v) = |c|,
    # so W' = W - lr c / (|c| + eps).  Catches sum-instead-of-mean, eps inside
    # the root, and a missing (1 - beta2).
    c = 3.0
    dim = 768
    G = np.full((1, dim), c, np.float32)
    W = np.full((1, dim), 0.5, np.float32)
    lr, eps = 0.01, 1e-3
    Wn, vn, tn = oracle.sparse_step(G, W, np.zeros(1, np.float32), np.zeros(1, np.int32),
                                    1, lr, 0.0, eps)
    assert vn[0] == np.float32(9.0)
    expect = 0.5 - float(np.float32(lr)) * c / (c + float(np.float32(eps)))
    assert Wn[0, 0] == np.float32(expect)
    assert tn[0] == 1


def test_decay_exponent_is_steps_missed():
    # beta2 = 0.5, touched at t = 1, then touched at t = 5 with a zero
    # gradient: v = 0.5^4 v1 exactly, W unchanged, t_last = 5.
    dim = 768
    G1 = np.full((1, dim), 2.0, np.float32)
    W = np.full((1, dim), 0.1, np.float32)
    W1, v1, t1 = oracle.sparse_step(G1, W, np.zeros(1, np.float32), np.zeros(1, np.int32),
                                    1, 0.01, 0.5, 1e-8)
    assert v1[0] == np.float32(0.5 * 4.0)
    W5, v5, t5 = oracle.sparse_step(np.zeros((1, dim), np.float32), W1, v1, t1, 5, 0.01,
                                    0.5, 1e-8)
    assert v5[0] == v1[0] / 16
    np.testing.assert_array_equal(W5, W1)
    assert t5[0] == 5


def test_sign_symmetry_and_scale_invariance():
    rs = np.random.default_rng(2)
    G = rs.standard_normal((3, 768)).astype(np.float32)
    W = rs.standard_normal((3, 768)).astype(np.float32)
    tl = np.zeros(3, np.int32)
    Wp, vp, _ = oracle.sparse_step(G, W, np.zeros(3, np.float32), tl, 1, 0.01, 0.95, 1e-12)
    Wm, vm, _ = oracle.sparse_step(-G, W, np.zeros(3, np.float32), tl, 1, 0.01, 0.95, 1e-12)
    np.testing.assert_array_equal(vp, vm)
    big = np.maximum(np.maximum(np.abs(W), np.abs(Wp)), np.abs(Wm))
    ulp = np.spacing(big).astype(np.float64)   # fp32 rounding of W' itself
    assert np.all(np.abs((Wp.astype(np.float64) - W) + (Wm.astype(np.float64) - W)) <= ulp)
    # Adam-style normalisation: scaling G (from v = 0) leaves the step unchanged
    W4, v4, _ = oracle.sparse_step(4 * G, W, np.zeros(3, np.float32), tl, 1, 0.01, 0.95, 1e-12)
    np.testing.assert_allclose(v4, 16 * vp, rtol=1e-6)
    assert np.all(np.abs(W4.astype(np.float64) - Wp) <= ulp)


@pytest.mark.parametrize("beta2", [0.0, 0.5, 0.95, 0.999])
def test_first_touch_from_zero_state(beta2):
    # from v = 0: v = (1 - beta2) mean(G^2) regardless of the decay exponent
    rs = np.random.default_rng(3)
    G = rs.standard_normal((2, 768)).astype(np.float32)
    W = np.zeros((2, 768), np.float32)
    _, va, _ = oracle.sparse_step(G, W, np.zeros(2, np.float32), np.zeros(2, np.int32),
                                  1, 0.01, beta2, 1e-8)
    _, vb, _ = oracle.sparse_step(G, W, np.zeros(2, np.float32), np.zeros(2, np.int32),
                                  9, 0.01, beta2, 1e-8)
    np.testing.assert_array_equal(va, vb)
    m = (G.astype(np.float64) ** 2).mean(axis=1)
    np.testing.assert_allclose(va, (1 - float(np.float32(beta2))) * m, rtol=1e-6)


def test_bf16_rows_round_once():
    # bf16 storage: W' is the fp64 update rounded once to bf16
    rs = np.random.default_rng(4)
    G = rs.standard_normal((4, 768)).astype(np.float32)
    Wf = (rs.standard_normal((4, 768)) * 0.02).astype(np.float32)
    Wbits = np.array([[oracle.double_to_bf16(float(x)) for x in r] for r in Wf], np.uint16)
    Wn, vn, _ = oracle.sparse_step(G, Wbits, np.zeros(4, np.float32), np.zeros(4, np.int32),
                                   1, 0.01, 0.95, 1e-8)
    Wf_in = (Wbits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    upd = 0.01 * G.astype(np.float64) / (np.sqrt(vn.astype(np.float64))[:, None]
                                         + float(np.float32(1e-8)))
    lr32 = float(np.float32(0.01))
    upd *= lr32 / 0.01
    for u in range(4):
        for d in range(0, 768, 97):
            assert Wn[u, d] == oracle.double_to_bf16(Wf_in[u, d] - upd[u, d])
