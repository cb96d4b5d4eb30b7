"""ngram_touched_rows: the window's distinct rows per channel, ascending (only
the rows that receive the window's update are passed on: the @classiclarryd
post quoted on the airebao.com item).  Compared element by element with
np.unique of the oracle's rows, in every mode, for rows already reduced into
the window, rows kept in the burst stash, and a mix of both; truncation to
max_rows keeps the first rows and the full count; a token-indexed table has
no second channel.  Full-size and graph-captured windows are checked in
test_gpu_full.py and test_gpu_graph.py."""
import numpy as np
import pytest
import torch

import helpers
from gpu_common import ng, to_dev, window_inputs
from sparse_hashed_gram_amd import synth, workloads

pytestmark = pytest.mark.gpu

W = workloads.TINY


def _expect(toks, c):
    return np.unique(np.concatenate([helpers.oracle_rows(W, t, W.rows)[2 * c] for t in toks]))


def _got(N, cfg, ws, c, max_rows=None):
    rows = None if max_rows is None else torch.empty(max_rows, dtype=torch.int32, device="cuda")
    r, n = N.touched_rows(cfg, ws, c, rows=rows)
    n = int(n.item())
    return r[:min(n, r.numel())].cpu().numpy().astype(np.int64), n


@pytest.mark.parametrize("keys_ahead", [False, True])
@pytest.mark.parametrize("mode", ["spread", "burst", "burst_ref"])
def test_touched_rows_ascending(mode, keys_ahead):
    N = ng()
    cfg = N.config(W.vocab, W.eos_id, W.rows, "f32", max_tokens=W.tokens_per_step, mode=mode)
    ws = N.Workspace(cfg)
    toks, dys = window_inputs(W, 0)
    keep = [to_dev(d) for d in dys]
    if keys_ahead and mode != "spread":   # keys recorded ahead, no gradients attached yet
        for t in toks:
            N.window_keys(cfg, ws, to_dev(t))
    else:
        for t, d in zip(toks, keep):
            N.embed_bwd_accum(cfg, ws, to_dev(t), d)
    for c in range(2):
        got, n = _got(N, cfg, ws, c)
        want = _expect(toks, c)
        assert n == len(want)
        np.testing.assert_array_equal(got, want)
        # truncated: the first max_rows rows, the whole count
        got, n = _got(N, cfg, ws, c, max_rows=100)
        assert n == len(want)
        np.testing.assert_array_equal(got, want[:100])
    assert N.device_status(cfg, ws) == 0


def test_touched_rows_reduced_and_kept():
    # burst: two micro-steps reduced into the window, two more kept
    N = ng()
    cfg = N.config(W.vocab, W.eos_id, W.rows, "f32", max_tokens=W.tokens_per_step, mode="burst")
    ws = N.Workspace(cfg)
    toks, dys = window_inputs(W, 4)
    for m in range(4):
        N.embed_bwd_accum(cfg, ws, to_dev(toks[m]), to_dev(dys[m]))
        if m == 1:
            N.window_reduce(cfg, ws)
    for c in range(2):
        got, n = _got(N, cfg, ws, c)
        np.testing.assert_array_equal(got, _expect(toks, c))
    # after the step the window is empty
    st = [N.new_state(r) for r in W.rows]
    Wt = [to_dev(synth.init_rows(W, c, W.rows[c])) for c in range(2)]
    N.sparse_step(cfg, ws, Wt[0], Wt[1], st[0], st[1], 1, W.lr, W.beta2, W.eps)
    for c in range(2):
        assert _got(N, cfg, ws, c)[1] == 0
    assert N.device_status(cfg, ws) == 0


def test_touched_rows_token_indexed():
    N = ng()
    V = W.vocab
    cfg = N.config(V, W.eos_id, (V, 1), "f32", max_tokens=W.tokens_per_step, mode="burst_ref", direct=True)
    ws = N.Workspace(cfg)
    toks, dys = window_inputs(W, 0)
    keep = [to_dev(d) for d in dys]
    for t, d in zip(toks, keep):
        N.embed_bwd_accum(cfg, ws, to_dev(t), d)
    got, n = _got(N, cfg, ws, 0)
    np.testing.assert_array_equal(got, np.unique(np.concatenate(toks)))
    assert _got(N, cfg, ws, 1)[1] == 0
