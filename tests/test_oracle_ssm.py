"""Pins of the sampled-softmax oracle (``oracle/ssm.py``) against things it
does not compute itself: hand-derived candidate sets, torch's cross-entropy on
the full vocabulary, torch autograd, central differences of the oracle's own
loss, and closed forms."""
import json
import os

import numpy as np
import pytest
import torch

from oracle import ssm

GOLD = os.path.join(os.path.dirname(__file__), "golden", "ssm_candidates.json")


def _case(seed, T=96, V=300, D=24, C=None, s=1.1):
    rs = np.random.default_rng(seed)
    p = np.arange(1, V + 1, dtype=np.float64) ** -s
    tgt = rs.choice(V, size=T, p=p / p.sum()).astype(np.int64)
    perm = rs.permutation(V)
    n = len(np.unique(tgt))
    C = C or min(V, n + 40)
    X = rs.standard_normal((T, D))
    W = rs.standard_normal((V, D)) * 0.3
    g = rs.standard_normal(T)
    return tgt, perm, X, W, g, C


# ------------------------------------------------------------ candidates

@pytest.mark.parametrize("k", range(5))
def test_candidates_golden(k):
    case = json.load(open(GOLD))["cases"][k]
    cand, slot, _, ok = ssm.candidates(np.array(case["targets"]), np.array(case["perm"]),
                                       case["vocab"], case["C"])
    assert ok == case["ok"]
    if ok:
        assert cand.tolist() == case["cand"]
        assert slot.tolist() == case["slot"]


@pytest.mark.parametrize("seed", range(6))
def test_candidate_set_properties(seed):
    tgt, perm, _, _, _, C = _case(seed, T=200, V=500)
    V = len(perm)
    cand, slot, n, ok = ssm.candidates(tgt, perm, V, C)
    assert ok and len(cand) == C and len(np.unique(cand)) == C
    assert np.array_equal(cand[slot], tgt)                         # every target is scored
    assert np.array_equal(cand[:n], np.unique(tgt))                # present ids first, ascending
    assert not np.isin(cand[n:], tgt).any()
    # the fill is a prefix of the permutation's absent ids: every chosen id
    # comes before every absent id that was not chosen
    pos = np.empty(V, np.int64)
    pos[perm] = np.arange(V)
    left_out = np.setdiff1d(np.arange(V), cand)
    if len(left_out) and C > n:
        assert pos[cand[n:]].max() < pos[left_out].min()
    assert np.all(np.diff(pos[cand[n:]]) > 0)


def test_full_vocabulary_is_a_permutation():
    tgt, perm, _, _, _, _ = _case(3, V=200)
    cand, _, _, ok = ssm.candidates(tgt, perm, 200, 200)
    assert ok and np.array_equal(np.sort(cand), np.arange(200))


# ------------------------------------------------------------------ loss

def test_full_vocabulary_loss_is_torch_cross_entropy():
    tgt, perm, X, W, _, _ = _case(1)
    V = len(W)
    cand, slot, _, _ = ssm.candidates(tgt, perm, V, V)
    loss, lse = ssm.loss_fwd(X, W, cand, slot, chunk=17)
    z = torch.from_numpy(X) @ torch.from_numpy(W).T                # vocabulary order
    ref = torch.nn.functional.cross_entropy(z, torch.from_numpy(tgt), reduction="none")
    np.testing.assert_allclose(loss, ref.numpy(), rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(lse, torch.logsumexp(z, 1).numpy(), rtol=1e-13, atol=1e-13)


def test_sampled_loss_is_cross_entropy_over_the_candidates():
    tgt, perm, X, W, _, C = _case(2)
    cand, slot, _, _ = ssm.candidates(tgt, perm, len(W), C)
    loss, _ = ssm.loss_fwd(X, W, cand, slot)
    zc = torch.from_numpy(X) @ torch.from_numpy(W[cand]).T
    ref = torch.nn.functional.cross_entropy(zc, torch.from_numpy(slot), reduction="none")
    np.testing.assert_allclose(loss, ref.numpy(), rtol=1e-13, atol=1e-13)


def test_loss_does_not_depend_on_candidate_order():
    tgt, perm, X, W, _, C = _case(4)
    cand, slot, _, _ = ssm.candidates(tgt, perm, len(W), C)
    sh = np.random.default_rng(0).permutation(C)
    inv = np.argsort(sh)
    l1, _ = ssm.loss_fwd(X, W, cand, slot)
    l2, _ = ssm.loss_fwd(X, W, cand[sh], inv[slot])
    np.testing.assert_allclose(l1, l2, rtol=1e-13, atol=1e-14)


def test_closed_forms():
    # two candidates with logits 0 and ln 3: loss of the first is ln 4
    X = np.array([[1.0, 0.0], [1.0, 0.0]])
    W = np.array([[0.0, 5.0], [np.log(3.0), -2.0]])
    loss, lse = ssm.loss_fwd(X, W, np.array([0, 1]), np.array([0, 1]))
    assert abs(lse[0] - np.log(4.0)) < 1e-15 and abs(loss[0] - np.log(4.0)) < 1e-15
    assert abs(loss[1] - (np.log(4.0) - np.log(3.0))) < 1e-15
    # W = 0: every loss is ln C, dX = 0, dW[c] = sum_i g_i (1/C - [c = slot_i]) X_i
    tgt, perm, X, W, g, C = _case(5)
    W0 = np.zeros_like(W)
    cand, slot, _, _ = ssm.candidates(tgt, perm, len(W), C)
    loss, _ = ssm.loss_fwd(X, W0, cand, slot)
    np.testing.assert_allclose(loss, np.log(C), rtol=1e-14)
    dX, dWc = ssm.loss_bwd(X, W0, cand, slot, g)
    assert np.abs(dX).max() == 0.0
    exp = np.outer(np.full(C, 1.0 / C), g @ X)
    for i in range(len(tgt)):
        exp[slot[i]] -= g[i] * X[i]
    np.testing.assert_allclose(dWc, exp, rtol=1e-12, atol=1e-12)
    # a single candidate: loss 0 and no gradient
    cand1, slot1, _, ok = ssm.candidates(np.full(5, 7), np.arange(20), 20, 1)
    assert ok
    Xs = np.random.default_rng(0).standard_normal((5, 4))
    Ws = np.random.default_rng(1).standard_normal((20, 4))
    l1, _ = ssm.loss_fwd(Xs, Ws, cand1, slot1)
    d1, w1 = ssm.loss_bwd(Xs, Ws, cand1, slot1, np.ones(5))
    assert np.abs(l1).max() < 1e-15 and np.abs(d1).max() < 1e-15 and np.abs(w1).max() < 1e-15


# -------------------------------------------------------------- backward

def test_backward_is_torch_autograd():
    tgt, perm, X, W, g, C = _case(6)
    cand, slot, _, _ = ssm.candidates(tgt, perm, len(W), C)
    dX, dWc = ssm.loss_bwd(X, W, cand, slot, g)
    Xt = torch.from_numpy(X).requires_grad_()
    Wt = torch.from_numpy(W).requires_grad_()
    z = Xt @ Wt[torch.from_numpy(cand)].T
    l = torch.nn.functional.cross_entropy(z, torch.from_numpy(slot), reduction="none")
    (l * torch.from_numpy(g)).sum().backward()
    np.testing.assert_allclose(dX, Xt.grad.numpy(), rtol=1e-12, atol=1e-13)
    full = np.zeros_like(W)
    full[cand] = dWc
    np.testing.assert_allclose(full, Wt.grad.numpy(), rtol=1e-12, atol=1e-13)


def test_backward_matches_central_differences():
    tgt, perm, X, W, g, C = _case(7, T=12, V=40, D=5)
    cand, slot, _, _ = ssm.candidates(tgt, perm, len(W), C)
    dX, dWc = ssm.loss_bwd(X, W, cand, slot, g)

    def L(Xv, Wv):
        return float(g @ ssm.loss_fwd(Xv, Wv, cand, slot)[0])

    h = 1e-6
    rs = np.random.default_rng(0)
    for _ in range(12):
        i, d = rs.integers(len(X)), rs.integers(X.shape[1])
        Xp, Xm = X.copy(), X.copy()
        Xp[i, d] += h
        Xm[i, d] -= h
        assert abs((L(Xp, W) - L(Xm, W)) / (2 * h) - dX[i, d]) < 1e-7
        c = rs.integers(C)
        Wp, Wm = W.copy(), W.copy()
        Wp[cand[c], d] += h
        Wm[cand[c], d] -= h
        assert abs((L(X, Wp) - L(X, Wm)) / (2 * h) - dWc[c, d]) < 1e-7


def test_dlogits_rows_sum_to_zero():
    # softmax minus one-hot: every position's dz sums to zero over the set
    tgt, perm, X, W, g, C = _case(8)
    cand, slot, _, _ = ssm.candidates(tgt, perm, len(W), C)
    dz = ssm.dlogits(X, W, cand, slot, g)
    np.testing.assert_allclose(dz.sum(1), 0.0, atol=1e-13)
    assert np.all(np.sign(dz[np.arange(len(tgt)), slot]) == -np.sign(g))


def test_dW_rows_are_torch_autograd_rows():
    # the sampled-row form used at full size, against autograd of the loss
    tgt, perm, X, W, g, C = _case(9)
    cand, slot, _, _ = ssm.candidates(tgt, perm, len(W), C)
    _, lse = ssm.loss_fwd(X, W, cand, slot)
    cs = np.array([0, 3, C // 2, C - 1])
    rows = ssm.dW_rows(X, W, cand, slot, g, lse, cs)
    Wt = torch.from_numpy(W).requires_grad_()
    z = torch.from_numpy(X) @ Wt[torch.from_numpy(cand)].T
    l = torch.nn.functional.cross_entropy(z, torch.from_numpy(slot), reduction="none")
    (l * torch.from_numpy(g)).sum().backward()
    np.testing.assert_allclose(rows, Wt.grad.numpy()[cand[cs]], rtol=1e-12, atol=1e-13)
