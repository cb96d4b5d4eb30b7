"""HIP-graph capture of whole accumulation windows (the speedrun captures its
training step in a graph: agentic-affairs "NanoGPT Training Record", ablation
section).  One window -- 4 x (forward, backward) and the sparse step, with
its step number and learning rate in device memory (the _dev step entry
points) -- is captured once and replayed for several windows, with new
tokens, gradients and step parameters copied into the captured buffers
between replays.  Every replay must equal the same window run eagerly through
the host-scalar entry points, bitwise: the same kernels on the same inputs,
and every replayed window is also checked against the oracle (touched sets
and t_last exact, v and W within tolerance, untouched rows unchanged).
Eager work and synchronisations run between the replays."""
import numpy as np
import pytest
import torch

from gpu_common import (State, check_step_against_oracle, ng, oracle_snapshots, to_dev, window_inputs,
                        window_oracle)
from sparse_hashed_gram_amd import synth, workloads

pytestmark = pytest.mark.gpu


def _tiny_state(cfg, w):
    return State(cfg, to_dev(synth.init_rows(w, 0, w.rows[0])),
                 to_dev(synth.init_rows(w, 1, w.rows[1])))


def _window_eager(N, cfg, st, ws, toks, dys, t, lr, beta2, eps, how):
    outs = []
    A = len(toks)
    for m in range(A):
        outs.append(N.embed_fwd(cfg, st.W[0], st.W[1], toks[m], ws=ws))
        if how == "fused_last" and m == A - 1:
            st.bwd_step(ws, toks[m], dys[m], t, lr, beta2, eps)
        else:
            N.embed_bwd_accum(cfg, ws, toks[m], dys[m])
    if how == "step":
        st.step(ws, t, lr, beta2, eps)
    return outs


@pytest.mark.parametrize("mode,how,nest", [(m, h, False) for m in ("spread", "burst", "burst_ref")
                                           for h in ("fused_last", "step")]
                         + [("burst_ref", "step", True), ("spread", "fused_last", True)])
def test_graph_replay_equals_eager(mode, how, nest):
    w = workloads.TINY
    N = ng()
    T, A = w.tokens_per_step, w.accum_steps
    cfg = N.config(w.vocab, w.eos_id, w.rows, "f32", max_tokens=T, mode=mode, nest_always=nest)
    eager = _tiny_state(cfg, w)
    graph = eager.clone()
    ws_e, ws_g = N.Workspace(cfg), N.Workspace(cfg)
    tok_s = [torch.zeros(T, dtype=torch.int32, device="cuda") for _ in range(A)]
    dy_s = [torch.zeros((T, 768), dtype=torch.float32, device="cuda") for _ in range(A)]
    out_s = [torch.empty((T, 768), dtype=torch.float32, device="cuda") for _ in range(A)]
    params = N.step_params(1, w.lr, w.beta2, w.eps)
    trows = [torch.empty(A * T, dtype=torch.int32, device="cuda") for _ in range(2)]
    tcount = [torch.empty(1, dtype=torch.int64, device="cuda") for _ in range(2)]
    torch.cuda.synchronize()

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for m in range(A):
            N.embed_fwd(cfg, graph.W[0], graph.W[1], tok_s[m], out=out_s[m], ws=ws_g)
            if how == "fused_last" and m == A - 1:
                N.embed_bwd_step_dev(cfg, ws_g, tok_s[m], dy_s[m], graph.W[0], graph.W[1], graph.st[0],
                                     graph.st[1], params)
            else:
                N.embed_bwd_accum(cfg, ws_g, tok_s[m], dy_s[m])
        if how == "step":
            for c in range(2):   # the window's rows, ascending, captured with the rest
                N.touched_rows(cfg, ws_g, c, rows=trows[c], count=tcount[c])
            N.sparse_step_dev(cfg, ws_g, graph.W[0], graph.W[1], graph.st[0], graph.st[1], params)

    for win in range(3):
        toks_np, dys_np = window_inputs(w, 4 * win)
        toks = [to_dev(x) for x in toks_np]
        dys = [to_dev(x) for x in dys_np]
        t, lr = win + 1, w.lr * (1.0 - 0.25 * win)   # a new step number and learning rate each window
        for m in range(A):
            tok_s[m].copy_(toks[m])
            dy_s[m].copy_(dys[m])
        N.step_params(t, lr, w.beta2, w.eps, out=params)
        snaps = oracle_snapshots(graph, window_oracle(cfg, toks_np, dys_np), np.random.default_rng(win))
        g.replay()
        outs = _window_eager(N, cfg, eager, ws_e, toks, dys, t, lr, w.beta2, w.eps, how)
        torch.cuda.synchronize()
        check_step_against_oracle(graph, snaps, t, lr, w.beta2, w.eps, "f32")
        if how == "step":
            for c in range(2):
                want = snaps[c]["touched"]
                assert int(tcount[c].item()) == len(want)
                np.testing.assert_array_equal(trows[c][:len(want)].cpu().numpy().astype(np.int64), want)
        for m in range(A):
            assert torch.equal(out_s[m], outs[m]), f"window {win}: forward {m} differs"
        for c in range(2):
            assert torch.equal(graph.W[c], eager.W[c]), f"window {win}: table {c} differs"
            assert torch.equal(graph.st[c], eager.st[c]), f"window {win}: row state {c} differs"
        assert int((eager.tl[0] == t).sum()) > 0
        # unrelated eager work between replays
        junk = torch.randn(1 << 16, device="cuda").sum()
        torch.cuda.synchronize()
        del junk
    assert N.device_status(cfg, ws_g) == 0
    assert N.device_status(cfg, ws_e) == 0


@pytest.mark.parametrize("mode", ["spread", "burst_ref"])
@pytest.mark.parametrize("bad", [(0, 0.01, 0.95, 1e-8), (1, 0.01, 1.0, 1e-8), (1, 0.01, 0.95, 0.0),
                                 (1, float("nan"), 0.95, 1e-8)])
def test_bad_device_params_write_nothing(mode, bad):
    # out-of-range step parameters in device memory: the step changes no
    # table row and no row state, flags it, and still empties the window
    w = workloads.TINY
    N = ng()
    T = 512
    cfg = N.config(w.vocab, w.eos_id, w.rows, "f32", max_tokens=T, mode=mode)
    st = _tiny_state(cfg, w)
    before = st.clone()
    ws = N.Workspace(cfg)
    toks, dys = window_inputs(w, 0, T=T)
    keep = [to_dev(d) for d in dys]
    for tok, dy in zip(toks, keep):
        N.embed_bwd_accum(cfg, ws, to_dev(tok), dy)
    params = N.step_params(*bad)
    N.sparse_step_dev(cfg, ws, st.W[0], st.W[1], st.st[0], st.st[1], params)
    flags = N.device_status(cfg, ws, clear=True)
    assert flags & N.FLAG_BAD_PARAMS
    for c in range(2):
        assert torch.equal(st.W[c], before.W[c])
        assert torch.equal(st.st[c], before.st[c])
        r, _ = N.window_export(cfg, ws, c, with_grad=False)
        assert len(r) == 0
    # a good step afterwards works on a fresh window
    for tok, dy in zip(toks, keep):
        N.embed_bwd_accum(cfg, ws, to_dev(tok), dy)
    N.sparse_step_dev(cfg, ws, st.W[0], st.W[1], st.st[0], st.st[1], N.step_params(1, w.lr, w.beta2, w.eps))
    assert N.device_status(cfg, ws) == 0
    assert int((st.tl[0] == 1).sum()) > 0
    assert np.any(st.W[0].cpu().numpy() != before.W[0].cpu().numpy())
