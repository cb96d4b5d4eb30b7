"""Non-finite upstream gradients through every mode and every step path.

The pages fix nothing for NaN or Inf; the reading taken on both sides is that
they propagate like any other value: a window gradient holding +Inf gives
v = Inf, so the row's factor lr / (sqrt(v) + eps) is 0 and its finite
elements keep their value while the Inf element becomes 0 * Inf = NaN; a NaN
element (or +Inf and -Inf meeting in one element) makes v NaN and the whole
row NaN.  A bf16 NaN is written as 0x7FC0 on both sides.

A few positions of the tiny workload's first window get a NaN, +Inf or -Inf
in one element of their dY row: one of them on the hottest bigram row (a
segment long enough for the fix-up of partial rows), and one -Inf on the row
of an earlier +Inf in the same element (the two meet as NaN).  Every row
these positions reach must equal the oracle's bit for bit (fp32: the same
NaN elements and the same bits elsewhere); all other touched rows are held
to the usual tolerance; touched sets and t_last are exact.

Paths: the standalone step over an exported window ("export": spread, or a
burst window reduced ahead of the step), the step fused into the last
micro-step's reduction ("fused_last", with the rest of a spread window going
through the standalone step), and the burst window's whole reduction fused
with the step ("step"); fp32 and bf16 tables; fp32 and bf16 dY.
"""
import numpy as np
import pytest
import torch

import helpers
from gpu_common import (State, check_step_against_oracle, dy_dev, host_rows, host_vec, ng,
                        oracle_snapshots, round_to_bf16, to_dev, window_inputs, window_oracle)
from sparse_hashed_gram_amd import synth, workloads

pytestmark = pytest.mark.gpu

W = workloads.TINY


def _poisoned_window(cfg):
    """The tiny workload's first window with non-finite dY entries, and the
    positions (micro-step, index) that carry them."""
    toks, dys = window_inputs(W, 0)
    dys = [d.copy() for d in dys]
    rows = [helpers.oracle_rows(W, t, W.rows) for t in toks]
    rb = np.concatenate([r[0] for r in rows])
    T = W.tokens_per_step
    u, cnt = np.unique(rb, return_counts=True)
    hot = u[np.argmax(cnt)]
    hot_pos = int(np.flatnonzero(rb == hot)[-1])       # a late key of the longest bigram segment
    b_inf = rb[1 * T + 20]
    same = np.flatnonzero(rb == b_inf)
    later = int(same[same > 1 * T + 20][0]) if np.any(same > 1 * T + 20) else None
    marks = [(0, 10, 5, np.nan), (1, 20, 17, np.inf), (3, 30, 100, -np.inf),
             (hot_pos // T, hot_pos % T, 200, np.nan)]
    if later is not None:
        marks.append((later // T, later % T, 17, -np.inf))
    for m, i, d, val in marks:
        dys[m][i, d] = val
    return toks, dys, rows, marks


def _touched_by(rows, marks):
    """Rows of each channel that a poisoned position reaches."""
    out = []
    for c in range(2):
        out.append(np.unique([rows[m][2 * c][i] for m, i, _, _ in marks]))
    return out


def _same_bits(got, want, dtype):
    if dtype == "bf16":
        np.testing.assert_array_equal(got, want)
        return
    gn, wn = np.isnan(got), np.isnan(want)
    np.testing.assert_array_equal(gn, wn)
    np.testing.assert_array_equal(got[~gn].view(np.uint32), want[~wn].view(np.uint32))


def _same_class(got, want):
    """Non-finite values in the same places with the same sign of Inf; the
    finite ones within the v tolerance."""
    np.testing.assert_array_equal(np.isnan(got), np.isnan(want))
    np.testing.assert_array_equal(np.isposinf(got), np.isposinf(want))
    np.testing.assert_array_equal(np.isneginf(got), np.isneginf(want))


@pytest.mark.parametrize("dtype,dy_dtype", [("f32", "f32"), ("bf16", "f32"), ("bf16", "bf16")])
@pytest.mark.parametrize("mode,how,nest", [("spread", "export", False), ("spread", "fused_last", False),
                                           ("burst", "export", False), ("burst", "step", False),
                                           ("burst", "fused_last", False), ("burst_ref", "export", False),
                                           ("burst_ref", "step", False), ("burst_ref", "fused_last", False),
                                           ("burst_ref", "step", True), ("spread", "fused_last", True)])
def test_nonfinite_gradients_propagate(mode, how, nest, dtype, dy_dtype):
    N = ng()
    cfg = N.config(W.vocab, W.eos_id, W.rows, dtype, max_tokens=W.tokens_per_step, mode=mode,
                   dy_dtype=dy_dtype, nest_always=nest)
    tdt = torch.float32 if dtype == "f32" else torch.bfloat16
    st = State(cfg, to_dev(synth.init_rows(W, 0, W.rows[0])).to(tdt),
               to_dev(synth.init_rows(W, 1, W.rows[1])).to(tdt))
    ws = N.Workspace(cfg)
    toks, dys, rows, marks = _poisoned_window(cfg)
    if dy_dtype == "bf16":
        dys = [round_to_bf16(d) for d in dys]   # NaN and +-Inf are bf16 values too
    poisoned = _touched_by(rows, marks)
    orc = window_oracle(cfg, toks, dys)
    for c in range(2):   # the oracle itself: the poisoned rows carry the non-finite sums
        assert not np.isfinite(orc[c][1][np.isin(orc[c][0], poisoned[c])]).all(axis=1).any()
    snaps = oracle_snapshots(st, orc, np.random.default_rng(0))
    keep = [dy_dev(d, dy_dtype) for d in dys]
    last = len(toks) - 1 if how == "fused_last" else len(toks)
    for m in range(last):
        N.embed_bwd_accum(cfg, ws, to_dev(toks[m]), keep[m])
    t = 1
    if how == "export":
        N.window_reduce(cfg, ws)
        for c in range(2):
            r_g, G_g = N.window_export(cfg, ws, c)
            order = torch.argsort(r_g)
            r_g, G_g = r_g[order].cpu().numpy(), G_g[order].cpu().numpy()
            touched, G_o, A_o = orc[c]
            np.testing.assert_array_equal(r_g, touched)
            bad = np.isin(touched, poisoned[c])
            _same_class(G_g[bad], G_o[bad])
            fin = np.isfinite(G_o[bad])
            helpers.assert_grad_close(G_g[bad][fin], G_o[bad][fin], A_o[bad][fin])
            helpers.assert_grad_close(G_g[~bad], G_o[~bad], A_o[~bad])
        st.step(ws, t, W.lr, W.beta2, W.eps)
    elif how == "fused_last":
        st.bwd_step(ws, to_dev(toks[-1]), keep[-1], t, W.lr, W.beta2, W.eps)
    else:
        st.step(ws, t, W.lr, W.beta2, W.eps)
    res = check_step_against_oracle(st, snaps, t, W.lr, W.beta2, W.eps, dtype, skip=poisoned)
    for c in range(2):
        s = snaps[c]
        bad = np.isin(s["touched"], poisoned[c])
        assert bad.sum() == len(poisoned[c])
        W_o, v_o = res[c]
        _same_bits(host_rows(st.W[c], s["touched"][bad]), W_o[bad], dtype)
        v_g = host_vec(st.v[c], s["touched"][bad])
        _same_class(v_g, v_o[bad])
        assert not np.isfinite(v_o[bad]).any()   # every poisoned row's v is NaN or Inf
    assert N.device_status(cfg, ws) == 0
