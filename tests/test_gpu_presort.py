"""GPU checks of keys kept ahead and the presorted burst step.

A window's n-gram rows depend only on its tokens, so in the burst modes its
sort keys can be kept (ngram_window_keys) and sorted (ngram_window_sort)
before any gradient exists, e.g. on a second stream while the forwards run;
the backward then only attaches the gradients.  The results must be bitwise
those of the regular path (the same keys at the same stash positions, the
same sort, the same sums), which the other GPU tests hold to the oracle.  A
window that is not ready when it is reduced (keys without gradients, not
sorted since its last keys) must be dropped without changing any row.  The
windows taken ahead are also checked against the oracle directly.
"""
import numpy as np
import pytest
import torch

from gpu_common import (State, check_step_against_oracle, ng, oracle_snapshots, to_dev, window_inputs,
                        window_oracle)
from sparse_hashed_gram_amd import synth, workloads

pytestmark = pytest.mark.gpu

W = workloads.TINY


def _state(cfg):
    return State(cfg, to_dev(synth.init_rows(W, 0, W.rows[0])), to_dev(synth.init_rows(W, 1, W.rows[1])))


def _regular_window(N, cfg, st, ws, toks, dys, t, how):
    for m in range(len(toks)):
        if how == "fused_last" and m == len(toks) - 1:
            st.bwd_step(ws, toks[m], dys[m], t, W.lr, W.beta2, W.eps)
            return
        N.embed_bwd_accum(cfg, ws, toks[m], dys[m])
    st.step(ws, t, W.lr, W.beta2, W.eps)


def _ahead_window(N, cfg, st, ws, toks, dys, t, how, n_ahead, side):
    # keys (and, with presort, the sort) on a side stream, gradients on the main one
    main = torch.cuda.current_stream()
    side.wait_stream(main)
    with torch.cuda.stream(side):
        for m in range(n_ahead):
            N.window_keys(cfg, ws, toks[m])
        if cfg.options & N.OPT_PRESORT:
            N.window_sort(cfg, ws)
    main.wait_stream(side)
    _regular_window(N, cfg, st, ws, toks, dys, t, how)


@pytest.mark.parametrize("nest", [False, True])
@pytest.mark.parametrize("how", ["step", "fused_last"])
@pytest.mark.parametrize("presort", [False, True])
@pytest.mark.parametrize("mode", ["burst", "burst_ref"])
def test_keys_ahead_equal_the_regular_path(mode, presort, how, nest):
    N = ng()
    T = W.tokens_per_step
    cfg_r = N.config(W.vocab, W.eos_id, W.rows, "f32", max_tokens=T, mode=mode, nest_always=nest)
    cfg_a = N.config(W.vocab, W.eos_id, W.rows, "f32", max_tokens=T, mode=mode, presort=presort,
                     nest_always=nest)
    reg, ahd = _state(cfg_r), _state(cfg_a)
    ws_r, ws_a = N.Workspace(cfg_r), N.Workspace(cfg_a)
    side = torch.cuda.Stream()
    for win in range(2):
        toks_np, dys_np = window_inputs(W, 4 * win)
        toks = [to_dev(x) for x in toks_np]
        dys = [to_dev(x) for x in dys_np]
        snaps = oracle_snapshots(ahd, window_oracle(cfg_a, toks_np, dys_np), np.random.default_rng(win))
        _regular_window(N, cfg_r, reg, ws_r, toks, dys, win + 1, how)
        _ahead_window(N, cfg_a, ahd, ws_a, toks, dys, win + 1, how, 4, side)
        torch.cuda.synchronize()
        for c in range(2):
            assert torch.equal(reg.W[c], ahd.W[c]), (win, c)
            assert torch.equal(reg.st[c], ahd.st[c]), (win, c)
        check_step_against_oracle(ahd, snaps, win + 1, W.lr, W.beta2, W.eps, "f32")
    assert N.device_status(cfg_a, ws_a) == 0


@pytest.mark.parametrize("mode", ["burst", "burst_ref"])
def test_some_keys_ahead_ragged(mode):
    # keys ahead for the first two micro-steps only; ragged T
    N = ng()
    Ts = [64, 97, 1, 33]
    cfg_r = N.config(W.vocab, W.eos_id, W.rows, "f32", max_tokens=97, mode=mode)
    reg, ahd = _state(cfg_r), _state(cfg_r)
    ws_r, ws_a = N.Workspace(cfg_r), N.Workspace(cfg_r)
    side = torch.cuda.Stream()
    for win in range(3):
        toks = [to_dev(synth.tokens(W, 300 + 4 * win + m, Ts[m])) for m in range(4)]
        dys = [to_dev(synth.dY(W, 300 + 4 * win + m, Ts[m])) for m in range(4)]
        toks_np = [synth.tokens(W, 300 + 4 * win + m, Ts[m]) for m in range(4)]
        dys_np = [synth.dY(W, 300 + 4 * win + m, Ts[m]) for m in range(4)]
        snaps = oracle_snapshots(ahd, window_oracle(cfg_r, toks_np, dys_np), np.random.default_rng(win))
        _regular_window(N, cfg_r, reg, ws_r, toks, dys, win + 1, "step")
        _ahead_window(N, cfg_r, ahd, ws_a, toks, dys, win + 1, "step", 2, side)
        torch.cuda.synchronize()
        for c in range(2):
            assert torch.equal(reg.W[c], ahd.W[c]) and torch.equal(reg.st[c], ahd.st[c])
        check_step_against_oracle(ahd, snaps, win + 1, W.lr, W.beta2, W.eps, "f32")
    assert N.device_status(cfg_r, ws_a) == 0


def _dropped(N, cfg, st, ws, before, flag):
    torch.cuda.synchronize()
    f = N.device_status(cfg, ws, clear=True)
    assert f & flag, hex(f)
    for c in range(2):
        assert torch.equal(st.W[c], before.W[c])
        assert torch.equal(st.st[c], before.st[c])


@pytest.mark.parametrize("case", ["not_sorted", "keys_after_sort", "missing_gradients", "t_mismatch"])
def test_unready_windows_are_dropped(case):
    N = ng()
    T = 256
    cfg = N.config(W.vocab, W.eos_id, W.rows, "f32", max_tokens=T, mode="burst_ref",
                   presort=case in ("not_sorted", "keys_after_sort"))
    st = _state(cfg)
    before = st.clone()
    ws = N.Workspace(cfg)
    toks_np, dys_np = window_inputs(W, 0, T=T)
    toks = [to_dev(x) for x in toks_np]
    dys = [to_dev(x) for x in dys_np]
    if case == "not_sorted":
        for m in range(4):
            N.embed_bwd_accum(cfg, ws, toks[m], dys[m])
    elif case == "keys_after_sort":
        for m in range(3):
            N.window_keys(cfg, ws, toks[m])
        N.window_sort(cfg, ws)
        N.window_keys(cfg, ws, toks[3])
        for m in range(4):
            N.embed_bwd_accum(cfg, ws, toks[m], dys[m])
    elif case == "missing_gradients":
        for m in range(4):
            N.window_keys(cfg, ws, toks[m])
        for m in range(3):
            N.embed_bwd_accum(cfg, ws, toks[m], dys[m])
    else:
        for m in range(4):
            N.window_keys(cfg, ws, toks[m])
        N.embed_bwd_accum(cfg, ws, toks[0], dys[0])
        N.embed_bwd_accum(cfg, ws, toks[1][:100].contiguous(), dys[1][:100].contiguous())
        assert N.device_status(cfg, ws) & N.FLAG_KEYS_MISMATCH
    st.step(ws, 1, W.lr, W.beta2, W.eps)
    _dropped(N, cfg, st, ws, before, N.FLAG_WINDOW_UNREADY)
    # the window is empty afterwards and the next one is stepped normally
    if cfg.options & N.OPT_PRESORT:
        for m in range(4):
            N.window_keys(cfg, ws, toks[m])
        N.window_sort(cfg, ws)
    for m in range(4):
        N.embed_bwd_accum(cfg, ws, toks[m], dys[m])
    st.step(ws, 1, W.lr, W.beta2, W.eps)
    torch.cuda.synchronize()
    assert N.device_status(cfg, ws) == 0
    assert int((st.tl[0] == 1).sum()) > 0
    assert np.any(st.W[0].cpu().numpy() != before.W[0].cpu().numpy())
