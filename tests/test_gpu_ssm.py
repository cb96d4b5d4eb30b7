"""GPU parity of the sampled-softmax loss (include/ssm.h) against the fp64
oracle (oracle/ssm.py), through the C ABI.

The candidate set and the slots are integer work: bit-exact.  Losses and
gradients are floating point; their tolerances are derived from the
arithmetic of the HIP path and written out below:

* logits: exact bf16 x bf16 products summed in fp32 over k = 768, so
  |dz_logit| <= 768 u sum_k |x_k w_k| (u = 2^-24), any summation order;
* lse: the largest logit error, plus the fp32 sums of exp over the tile and
  over the tiles (at most 66 + C/128 roundings of a positive sum) and the
  exp/log evaluations: (C/128 + 128) 2^-23 + 2^-22 |lse|;
* between the forward and the backward each logit is kept as q = exp(z - M) in
  fp16, M its row's maximum over the forward's column tile: q lies in (0, 1],
  so the rounding is within 2^-11 relative (2^-25 absolute below 2^-14);
* dz = g (q exp(M - lse) - onehot) is rounded to bf16 (2^-8 relative: an
  8-bit significand) after an fp32 evaluation whose error is
  g p (logit error + lse error + 2^-18 + 2^-11) + g 2^-25 (two fast exps of
  arguments whose size matters only while p is not negligible, one product,
  and q's rounding);
* dX = dz W_S and dW = dz^T X: exact products of bf16 values summed in fp32
  over K = C (or T) padded to 128, so each entry is off by at most
  sum |d(dz)| |w| + K u sum |dz w|, with d(dz) the bound above.
"""
import numpy as np
import pytest
import torch

from oracle import ssm as orc
from sparse_hashed_gram_amd import synth

pytestmark = pytest.mark.gpu

U = 2.0 ** -24
V_SMALL = 3000


def S():
    from sparse_hashed_gram_amd import ssm
    return ssm


def bf16_round(a: np.ndarray) -> np.ndarray:
    return torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(torch.bfloat16).float().numpy()


def _inputs(step, T, V):
    tgt, X, W, perm, g = synth.ssm_inputs(step, T, V)
    return tgt, bf16_round(X), bf16_round(W), perm, g


def _dev_bf16(a):
    return torch.from_numpy(a).to(torch.bfloat16).cuda()


def _dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def _run_cand(N, V, C, T, tgt, perm):
    cfg = N.config(V, C, max(T, 1))
    ws = N.Workspace(cfg)
    cand, slot = N.candidates(cfg, ws, _dev(tgt), _dev(perm))
    return cfg, ws, cand, slot


def _logit_err(X, W, cand):
    """768 u sum_k |x_k w_k| per (position, candidate)."""
    return 768 * U * (np.abs(X.astype(np.float64)) @ np.abs(W[cand].astype(np.float64)).T)


def _lse_tol(lse, zerr_max, C):
    return zerr_max + (C / 128 + 128) * 2.0 ** -23 + 2.0 ** -22 * np.abs(lse)


def _dz_bound(X, W, cand, slot, g, lse_tol):
    """(|dz| of the oracle, the per-entry bound on the GPU's dz)."""
    zerr = _logit_err(X, W, cand)
    dz = orc.dlogits(X, W, cand, slot, g)
    z = orc.logits(X, W, cand)
    _, lse = orc.loss_fwd(X, W, cand, slot)
    p = np.exp(z - lse[:, None])
    g = np.asarray(g, np.float64)[:, None]
    e1 = (np.abs(g) * p * (zerr + lse_tol[:, None] + 2.0 ** -18 + 2.0 ** -11)   # fp32 evaluation, fp16 q
          + np.abs(g) * (U + 2.0 ** -25))
    return dz, e1 + 2.0 ** -8 * (np.abs(dz) + e1)                                  # then bf16 rounding


# ------------------------------------------------------------ candidates

@pytest.mark.parametrize("T,C", [(1, 1), (1, 50), (100, 1000), (2048, 3000), (5000, 2500), (333, 2999)])
def test_candidates_bit_exact(T, C):
    N = S()
    tgt, _, _, perm, _ = _inputs(T, T, V_SMALL)
    cand_o, slot_o, n, ok = orc.candidates(tgt, perm, V_SMALL, C)
    if not ok:
        C = n   # exactly as many candidates as distinct targets
        cand_o, slot_o, n, ok = orc.candidates(tgt, perm, V_SMALL, C)
    cfg, ws, cand, slot = _run_cand(N, V_SMALL, C, T, tgt, perm)
    assert np.array_equal(cand.cpu().numpy(), cand_o)
    assert np.array_equal(slot.cpu().numpy(), slot_o)
    assert N.device_status(cfg, ws) == 0


def test_candidates_full_size_and_full_vocabulary():
    N = S()
    V, T = 50304, 49152
    tgt, _, _, perm, _ = _inputs(0, T, V)
    for C in (10240, 14336, V):
        cand_o, slot_o, _, ok = orc.candidates(tgt, perm, V, C)
        assert ok
        cfg, ws, cand, slot = _run_cand(N, V, C, T, tgt, perm)
        assert np.array_equal(cand.cpu().numpy(), cand_o), C
        assert np.array_equal(slot.cpu().numpy(), slot_o), C
        assert N.device_status(cfg, ws) == 0


@pytest.mark.parametrize("case", ["no_forward", "other_T", "new_candidates"])
def test_backward_needs_its_forward(case):
    # dz comes from the logits the forward stored: a backward with no forward
    # since the candidate set, or with another T, gives zero gradients and
    # SSM_FLAG_NO_LOGITS; the workspace works again after a forward
    N = S()
    T, V, C = 400, V_SMALL, 500
    tgt, X, W, perm, g = _inputs(8, T, V)
    cfg, ws, cand, slot = _run_cand(N, V, C, T, tgt, perm)
    Xd, Wd = _dev_bf16(X), _dev_bf16(W)
    Tb = T
    if case == "other_T":
        N.loss_fwd(cfg, ws, Xd[:300], Wd, cand, slot[:300])
        Tb = 200
    elif case == "new_candidates":
        N.loss_fwd(cfg, ws, Xd, Wd, cand, slot)
        cand, slot = N.candidates(cfg, ws, _dev(tgt), _dev(perm))
    lse = torch.zeros(Tb, device="cuda")
    dW = torch.full((V, 768), 0.25, device="cuda")
    dX = N.loss_bwd(cfg, ws, Xd[:Tb], Wd, cand, slot[:Tb], lse, _dev(g[:Tb]), dW)
    assert torch.count_nonzero(dX) == 0 and bool((dW == 0.25).all())
    assert N.device_status(cfg, ws, clear=True) == N.FLAG_NO_LOGITS
    _, lse = N.loss_fwd(cfg, ws, Xd, Wd, cand, slot)
    dX = N.loss_bwd(cfg, ws, Xd, Wd, cand, slot, lse, _dev(g), dW)
    cand_o, slot_o, _, _ = orc.candidates(tgt, perm, V, C)
    dX_o, _ = orc.loss_bwd(X, W, cand_o, slot_o, g)
    assert np.abs(dX.cpu().numpy() - dX_o).max() <= 1e-2 * np.abs(dX_o).max()
    assert N.device_status(cfg, ws) == 0


@pytest.mark.parametrize("case", ["overflow", "bad_target", "bad_perm"])
def test_void_batches(case):
    N = S()
    T, V, C = 500, V_SMALL, 400
    tgt, X, W, perm, g = _inputs(7, T, V)
    flag = {"overflow": N.FLAG_OVERFLOW, "bad_target": N.FLAG_BAD_TARGET, "bad_perm": N.FLAG_BAD_PERM}[case]
    if case == "overflow":
        C = len(np.unique(tgt)) - 1
    elif case == "bad_target":
        tgt = tgt.copy()
        tgt[17] = V + 3
    else:
        perm = perm.copy()
        perm[5] = perm[6]
    cfg, ws, cand, slot = _run_cand(N, V, C, T, tgt, perm)
    c, sl = cand.cpu().numpy(), slot.cpu().numpy()
    assert c.min() >= 0 and c.max() < V and sl.min() >= 0 and sl.max() < C
    Xd, Wd = _dev_bf16(X), _dev_bf16(W)
    loss, lse = N.loss_fwd(cfg, ws, Xd, Wd, cand, slot)
    dW = torch.full((V, 768), 0.25, device="cuda")
    dX = N.loss_bwd(cfg, ws, Xd, Wd, cand, slot, lse, _dev(g), dW)
    assert torch.isnan(loss).all() and torch.isnan(lse).all()
    assert torch.count_nonzero(dX) == 0 and bool((dW == 0.25).all())
    assert N.device_status(cfg, ws, clear=True) & flag
    # a good batch on the same workspace works again
    tgt2 = np.arange(10, dtype=np.int32)
    perm2 = np.random.default_rng(1).permutation(V).astype(np.int32)
    cand2, slot2 = N.candidates(cfg, ws, _dev(tgt2), _dev(perm2))
    loss2, _ = N.loss_fwd(cfg, ws, _dev_bf16(X[:10]), Wd, cand2, slot2)
    assert torch.isfinite(loss2).all() and N.device_status(cfg, ws) == 0


# --------------------------------------------------------------- forward

def _check_fwd(X, W, cand_o, slot_o, loss, lse, C, rows=None):
    rows = np.arange(len(X)) if rows is None else rows
    Xs = X[rows]
    loss_o, lse_o = orc.loss_fwd(Xs, W, cand_o, slot_o[rows])
    zerr = _logit_err(Xs, W, cand_o)
    tl = _lse_tol(lse_o, zerr.max(axis=1), C)
    l_g = lse.cpu().numpy()[rows].astype(np.float64)
    s_g = loss.cpu().numpy()[rows].astype(np.float64)
    assert np.all(np.abs(l_g - lse_o) <= tl), np.max(np.abs(l_g - lse_o) / tl)
    tz = zerr[np.arange(len(rows)), slot_o[rows]]
    assert np.all(np.abs(s_g - loss_o) <= tl + tz), np.max(np.abs(s_g - loss_o) / (tl + tz))


# C in (128, 192]: the second 192-column tile lies wholly past C (its partial
# sums are (-inf, 0) and the lse fold skips them)
@pytest.mark.parametrize("T,C", [(1, 1), (1, 300), (77, 128), (77, 150), (130, 192), (300, 1000), (1000, 1290),
                                 (2000, 2999)])
def test_forward_matches_oracle(T, C):
    N = S()
    tgt, X, W, perm, _ = _inputs(100 + T, T, V_SMALL)
    C = max(C, len(np.unique(tgt)))
    cand_o, slot_o, _, _ = orc.candidates(tgt, perm, V_SMALL, C)
    cfg, ws, cand, slot = _run_cand(N, V_SMALL, C, T, tgt, perm)
    loss, lse = N.loss_fwd(cfg, ws, _dev_bf16(X), _dev_bf16(W), cand, slot)
    _check_fwd(X, W, cand_o, slot_o, loss, lse, C)
    assert N.device_status(cfg, ws) == 0


# -------------------------------------------------------------- backward

def _check_bwd(X, W, cand_o, slot_o, g, dX, dW, dW0, C):
    T = len(X)
    _, lse_o = orc.loss_fwd(X, W, cand_o, slot_o)
    zerr = _logit_err(X, W, cand_o)
    tl = _lse_tol(lse_o, zerr.max(axis=1), C)
    dz, e = _dz_bound(X, W, cand_o, slot_o, g, tl)
    Wc = np.abs(W[cand_o].astype(np.float64))
    Xa = np.abs(X.astype(np.float64))
    Kc, Kt = -(-C // 128) * 128, -(-T // 128) * 128
    dX_o = dz @ W[cand_o].astype(np.float64)
    tol_x = e @ Wc + Kc * U * (np.abs(dz) @ Wc) + 1e-30
    err = np.abs(dX.cpu().numpy().astype(np.float64) - dX_o)
    assert np.all(err <= tol_x), np.max(err / tol_x)
    dWc_o = dz.T @ X.astype(np.float64)
    got = dW.cpu().numpy().astype(np.float64)
    tol_w = e.T @ Xa + Kt * U * (np.abs(dz).T @ Xa) + U * np.abs(dW0[cand_o] + dWc_o) + 1e-30
    err = np.abs(got[cand_o] - (dW0[cand_o] + dWc_o))
    assert np.all(err <= tol_w), np.max(err / tol_w)
    rest = np.setdiff1d(np.arange(len(W)), cand_o)
    assert np.array_equal(got[rest], dW0[rest].astype(np.float64))   # untouched rows


@pytest.mark.parametrize("T,C", [(1, 1), (5, 300), (77, 128), (77, 150), (300, 1000), (1000, 1290), (2000, 2999)])
def test_backward_matches_oracle(T, C):
    N = S()
    tgt, X, W, perm, g = _inputs(200 + T, T, V_SMALL)
    C = max(C, len(np.unique(tgt)))
    cand_o, slot_o, _, _ = orc.candidates(tgt, perm, V_SMALL, C)
    cfg, ws, cand, slot = _run_cand(N, V_SMALL, C, T, tgt, perm)
    Xd, Wd = _dev_bf16(X), _dev_bf16(W)
    loss, lse = N.loss_fwd(cfg, ws, Xd, Wd, cand, slot)
    dW0 = np.random.default_rng(T).standard_normal((V_SMALL, 768)).astype(np.float32)
    dW = _dev(dW0)
    dX = N.loss_bwd(cfg, ws, Xd, Wd, cand, slot, lse, _dev(g), dW)
    _check_bwd(X, W, cand_o, slot_o, g, dX, dW, dW0, C)
    assert N.device_status(cfg, ws) == 0


def test_backward_accumulates_over_calls():
    # two micro-batches into one dW: the sum of both contributions
    N = S()
    T, C = 640, 1200
    dW = torch.zeros((V_SMALL, 768), device="cuda")
    ref = np.zeros((V_SMALL, 768))
    for step in (1, 2):
        tgt, X, W, perm, g = _inputs(300 + step, T, V_SMALL)
        cand_o, slot_o, _, _ = orc.candidates(tgt, perm, V_SMALL, C)
        cfg, ws, cand, slot = _run_cand(N, V_SMALL, C, T, tgt, perm)
        Xd, Wd = _dev_bf16(X), _dev_bf16(W)
        _, lse = N.loss_fwd(cfg, ws, Xd, Wd, cand, slot)
        N.loss_bwd(cfg, ws, Xd, Wd, cand, slot, lse, _dev(g), dW)
        ref[cand_o] += orc.loss_bwd(X, W, cand_o, slot_o, g)[1]
    got = dW.cpu().numpy()
    scale = np.abs(ref).max()
    assert np.abs(got - ref).max() <= 2e-3 * scale


def test_deterministic():
    N = S()
    T, C = 1500, 2000
    tgt, X, W, perm, g = _inputs(9, T, V_SMALL)
    outs = []
    for _ in range(2):
        cfg, ws, cand, slot = _run_cand(N, V_SMALL, C, T, tgt, perm)
        Xd, Wd = _dev_bf16(X), _dev_bf16(W)
        loss, lse = N.loss_fwd(cfg, ws, Xd, Wd, cand, slot)
        dW = torch.zeros((V_SMALL, 768), device="cuda")
        dX = N.loss_bwd(cfg, ws, Xd, Wd, cand, slot, lse, _dev(g), dW)
        outs.append((loss, lse, dX, dW))
    for a, b in zip(*outs):
        assert torch.equal(a, b)


# ------------------------------------------------------------- full size

@pytest.mark.parametrize("C", [10240, 50304])
def test_full_size_sampled(C):
    # one GPU's micro-batch (49,152 positions) against the whole vocabulary
    # table; the oracle checks sampled positions and sampled candidates
    N = S()
    V = 50304
    T = 49152 if C == 10240 else 8192
    tgt, X, W, perm, g = _inputs(11, T, V)
    cand_o, slot_o, _, ok = orc.candidates(tgt, perm, V, C)
    assert ok
    cfg, ws, cand, slot = _run_cand(N, V, C, T, tgt, perm)
    assert np.array_equal(cand.cpu().numpy(), cand_o)
    Xd, Wd = _dev_bf16(X), _dev_bf16(W)
    loss, lse = N.loss_fwd(cfg, ws, Xd, Wd, cand, slot)
    dW = torch.zeros((V, 768), device="cuda")
    dX = N.loss_bwd(cfg, ws, Xd, Wd, cand, slot, lse, _dev(g), dW)
    torch.cuda.synchronize()
    assert N.device_status(cfg, ws) == 0
    rs = np.random.default_rng(C)
    rows = np.unique(np.r_[rs.integers(0, T, 96), T - 1])
    _check_fwd(X, W, cand_o, slot_o, loss, lse, C, rows)
    # dX of the sampled positions (each depends on its own row only)
    Xs = X[rows]
    _, lse_s = orc.loss_fwd(Xs, W, cand_o, slot_o[rows])
    tl = _lse_tol(lse_s, _logit_err(Xs, W, cand_o).max(axis=1), C)
    dz, e = _dz_bound(Xs, W, cand_o, slot_o[rows], g[rows], tl)
    Wc = np.abs(W[cand_o].astype(np.float64))
    Kc = -(-C // 128) * 128
    err = np.abs(dX.cpu().numpy()[rows].astype(np.float64) - dz @ W[cand_o].astype(np.float64))
    tol = e @ Wc + Kc * U * (np.abs(dz) @ Wc)
    assert np.all(err <= tol), np.max(err / tol)
    # dW of sampled candidates (each needs every position's lse): the hot
    # ids (most positions) and random ones, checked against a bound taken
    # with the largest per-position error factor
    _, lse_all = orc.loss_fwd(X, W, cand_o, slot_o)
    cs = np.unique(np.r_[np.arange(4), rs.integers(0, C, 12), C - 1])
    got = dW.cpu().numpy()[cand_o[cs]].astype(np.float64)
    exp = orc.dW_rows(X, W, cand_o, slot_o, g, lse_all, cs)
    Xa = np.abs(X.astype(np.float64))
    z = X.astype(np.float64) @ W[cand_o[cs]].astype(np.float64).T
    p = np.exp(z - lse_all[:, None])
    zerr = 768 * U * (Xa @ np.abs(W[cand_o[cs]].astype(np.float64)).T)
    # largest logit error of each position, by Cauchy-Schwarz: sum_k |x_k w_k| <= |x| max_c |w_c|
    zmax = 768 * U * np.linalg.norm(X.astype(np.float64), axis=1) * np.linalg.norm(
        W[cand_o].astype(np.float64), axis=1).max()
    lt = _lse_tol(lse_all, zmax, C)
    dzs = np.abs(g[:, None] * (p - (slot_o[:, None] == cs[None, :])))
    e1 = np.abs(g)[:, None] * p * (zerr + lt[:, None] + 2.0 ** -19) + np.abs(g)[:, None] * U
    e = e1 + 2.0 ** -8 * (dzs + e1)
    Kt = -(-T // 128) * 128
    tol = e.T @ Xa + Kt * U * (dzs.T @ Xa) + U * np.abs(exp)
    err = np.abs(got - exp)
    assert np.all(err <= tol), np.max(err / tol)
    # rows outside the candidate set stay zero
    out = np.setdiff1d(rs.integers(0, V, 4000), cand_o)[:500]
    assert not np.any(dW.cpu().numpy()[out])


def test_graph_replay_equals_eager():
    # candidate set, forward and backward captured once in a HIP graph and
    # replayed on new batches copied into the captured buffers; every replay
    # equals the same calls run eagerly, bitwise (dW accumulates in both)
    N = S()
    T, C, V = 1000, 1500, V_SMALL
    cfg = N.config(V, C, T)
    ws_g, ws_e = N.Workspace(cfg), N.Workspace(cfg)
    _, _, W, _, _ = _inputs(0, T, V)
    Wd = _dev_bf16(W)
    tgt_s = torch.zeros(T, dtype=torch.int32, device="cuda")
    perm_s = torch.zeros(V, dtype=torch.int32, device="cuda")
    X_s = torch.zeros((T, 768), dtype=torch.bfloat16, device="cuda")
    g_s = torch.zeros(T, dtype=torch.float32, device="cuda")
    cand_s = torch.empty(C, dtype=torch.int32, device="cuda")
    slot_s = torch.empty(T, dtype=torch.int32, device="cuda")
    loss_s = torch.empty(T, dtype=torch.float32, device="cuda")
    lse_s = torch.empty(T, dtype=torch.float32, device="cuda")
    dX_s = torch.empty((T, 768), dtype=torch.float32, device="cuda")
    dW_g = torch.zeros((V, 768), dtype=torch.float32, device="cuda")
    dW_e = torch.zeros((V, 768), dtype=torch.float32, device="cuda")
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        N.candidates(cfg, ws_g, tgt_s, perm_s, cand_s, slot_s)
        N.loss_fwd(cfg, ws_g, X_s, Wd, cand_s, slot_s, loss_s, lse_s)
        N.loss_bwd(cfg, ws_g, X_s, Wd, cand_s, slot_s, lse_s, g_s, dW_g, dX_s)
    for step in range(3):
        tgt, X, _, perm, g = _inputs(400 + step, T, V)
        tgt_s.copy_(_dev(tgt))
        perm_s.copy_(_dev(perm))
        X_s.copy_(_dev_bf16(X))
        g_s.copy_(_dev(g))
        graph.replay()
        cand, slot = N.candidates(cfg, ws_e, _dev(tgt), _dev(perm))
        loss, lse = N.loss_fwd(cfg, ws_e, _dev_bf16(X), Wd, cand, slot)
        dX = N.loss_bwd(cfg, ws_e, _dev_bf16(X), Wd, cand, slot, lse, _dev(g), dW_e)
        torch.cuda.synchronize()
        for a, b in ((cand_s, cand), (slot_s, slot), (loss_s, loss), (lse_s, lse), (dX_s, dX), (dW_g, dW_e)):
            assert torch.equal(a, b), f"replay {step} differs"
        junk = torch.randn(1 << 16, device="cuda").sum()   # unrelated eager work between replays
        torch.cuda.synchronize()
        del junk
    assert N.device_status(cfg, ws_g) == 0 and N.device_status(cfg, ws_e) == 0


def test_backward_dw_wide_tile_form():
    # 14,336 candidates: dW's 128 x 192 tiles (448 blocks in 512 slots) beat
    # the 128 x 128 ones (672 blocks, two rounds), so the library takes the
    # other dW form; same bar
    N = S()
    T, V, C = 700, 50304, 14336
    tgt, X, W, perm, g = _inputs(33, T, V)
    cand_o, slot_o, _, ok = orc.candidates(tgt, perm, V, C)
    assert ok
    cfg, ws, cand, slot = _run_cand(N, V, C, T, tgt, perm)
    Xd, Wd = _dev_bf16(X), _dev_bf16(W)
    loss, lse = N.loss_fwd(cfg, ws, Xd, Wd, cand, slot)
    dW0 = np.random.default_rng(5).standard_normal((V, 768)).astype(np.float32)
    dW = _dev(dW0)
    dX = N.loss_bwd(cfg, ws, Xd, Wd, cand, slot, lse, _dev(g), dW)
    _check_bwd(X, W, cand_o, slot_o, g, dX, dW, dW0, C)
    assert N.device_status(cfg, ws) == 0
