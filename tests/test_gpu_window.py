"""GPU parity of the backward (sort + dedupe + signed segment reduction with
4-step accumulation) and the lazy sparse row-wise step against the oracle,
in both the spread and the burst mode (amund.blog, The four improvements,
item 4), through the C ABI.

Tolerances: touched sets and t_last exact; window gradients per element
within 1e-5 of sum |s dY|; v within 1e-5 relative plus what that gradient
error can move (1 - beta2) mean(G^2); table rows within one ulp of the result
plus 1e-5 of the update plus the gradient error carried through
lr G / (sqrt(v) + eps) (which matters only where W - update cancels).
Untouched rows must stay bitwise unchanged.
"""
import numpy as np
import pytest
import torch

import helpers
from gpu_common import State, round_to_bf16, check_window, device_table, ng, to_dev, window_inputs
from sparse_hashed_gram_amd import synth, workloads

pytestmark = pytest.mark.gpu


def _tiny_state(cfg, w):
    return State(cfg, to_dev(synth.init_rows(w, 0, w.rows[0])),
                 to_dev(synth.init_rows(w, 1, w.rows[1])))


@pytest.mark.parametrize("mode", ["spread", "burst", "burst_ref"])
def test_tiny_workload_two_windows(mode):
    w = workloads.TINY
    N = ng()
    cfg = N.config(w.vocab, w.eos_id, w.rows, "f32", max_tokens=w.tokens_per_step, mode=mode)
    st = _tiny_state(cfg, w)
    ws = N.Workspace(cfg)
    for win in range(w.steps // w.accum_steps):
        toks, dys = window_inputs(w, win * w.accum_steps)
        check_window(st, ws, toks, dys, win + 1, w.lr, w.beta2, w.eps, "f32")
    assert N.device_status(cfg, ws) == 0


@pytest.mark.parametrize("nest", [False, True])
@pytest.mark.parametrize("mode,how", [("spread", "fused_last"), ("burst", "step"),
                                      ("burst", "fused_last"), ("spread", "step"),
                                      ("burst_ref", "step"), ("burst_ref", "fused_last")])
def test_tiny_workload_fused_step(mode, how, nest):
    # the step fused into the reduction: the last micro-step (spread) or the
    # whole window (burst); gradients are checked through the step results;
    # nest: with the nested sort, which windows this small skip by default
    w = workloads.TINY
    N = ng()
    cfg = N.config(w.vocab, w.eos_id, w.rows, "f32", max_tokens=w.tokens_per_step, mode=mode, nest_always=nest)
    st = _tiny_state(cfg, w)
    ws = N.Workspace(cfg)
    for win in range(w.steps // w.accum_steps):
        toks, dys = window_inputs(w, win * w.accum_steps)
        check_window(st, ws, toks, dys, win + 1, w.lr, w.beta2, w.eps, "f32", how=how)
    assert N.device_status(cfg, ws) == 0


@pytest.mark.parametrize("nest", [False, True])
@pytest.mark.parametrize("how", ["fused_last", "step"])
@pytest.mark.parametrize("mode", ["spread", "burst", "burst_ref"])
def test_shard_workload_fused(mode, how, nest):
    w = workloads.COLLISION
    N = ng()
    rows = workloads.SHARD.rows
    T = 49_152
    cfg = N.config(w.vocab, w.eos_id, rows, "bf16", max_tokens=T, mode=mode, nest_always=nest)
    st = State(cfg, device_table(rows[0], "bf16", 61), device_table(rows[1], "bf16", 62))
    ws = N.Workspace(cfg)
    for win in range(2):
        toks, dys = window_inputs(w, 4 * win, T=T)
        check_window(st, ws, toks, dys, win + 1, w.lr, w.beta2, w.eps, "bf16", how=how)
    assert N.device_status(cfg, ws) == 0
    del st, ws
    torch.cuda.empty_cache()


@pytest.mark.parametrize("nest", [False, True])
@pytest.mark.parametrize("T", [65, 129, 20_000])
def test_single_hot_row_fused(T, nest):
    w = workloads.TINY
    N = ng()
    cfg = N.config(w.vocab, w.eos_id, w.rows, "f32", max_tokens=T, nest_always=nest)
    st = _tiny_state(cfg, w)
    ws = N.Workspace(cfg)
    tok = np.full(T, 42, np.int32)
    dys = [synth.dY(w, 600 + m, T) for m in range(4)]
    check_window(st, ws, [tok] * 4, dys, 1, w.lr, w.beta2, w.eps, "f32", how="fused_last")


@pytest.mark.parametrize("mode", ["spread", "burst", "burst_ref"])
def test_small_table_long_gaps(mode):
    # 64-token micro-steps into 3000-row tables: rows skip windows, so the
    # retroactive beta2^k with k > 1 is exercised; ragged T per micro-step.
    w = workloads.TINY
    N = ng()
    rows = (2000, 3000)
    cfg = N.config(w.vocab, w.eos_id, rows, "f32", max_tokens=97, mode=mode)
    st = State(cfg, to_dev(synth.init_rows(w, 0, rows[0])), to_dev(synth.init_rows(w, 1, rows[1])))
    ws = N.Workspace(cfg)
    for win in range(8):
        Ts = [64, 97, 1, 33]
        toks = [synth.tokens(w, 100 + 4 * win + m, Ts[m]) for m in range(4)]
        dys = [synth.dY(w, 100 + 4 * win + m, Ts[m]) for m in range(4)]
        how = ("export", "fused_last", "step")[win % 3]
        check_window(st, ws, toks, dys, win + 1, 0.02, 0.9, 1e-6, "f32", how=how)
    gaps = st.tl[0].cpu().numpy()
    assert len(np.unique(gaps[gaps > 0])) > 3


@pytest.mark.parametrize("mode", ["spread", "burst"])
def test_shard_workload_bf16(mode):
    w = workloads.SHARD
    N = ng()
    cfg = N.config(w.vocab, w.eos_id, w.rows, "bf16", max_tokens=w.tokens_per_step, mode=mode)
    st = State(cfg, device_table(w.rows[0], "bf16", 21), device_table(w.rows[1], "bf16", 22))
    ws = N.Workspace(cfg)
    for win in range(3):
        toks, dys = window_inputs(w, 4 * win)
        check_window(st, ws, toks, dys, win + 1, w.lr, w.beta2, w.eps, "bf16")
    assert N.device_status(cfg, ws) == 0
    del st, ws
    torch.cuda.empty_cache()


def test_collision_skew_at_shard_scale():
    # Zipf 1.4 with 20% of tokens from a 256-id hot set: segments of thousands
    # of keys, so the cross-chunk partial sums and the fix-up pass are used.
    w = workloads.COLLISION
    N = ng()
    rows = workloads.SHARD.rows
    T = 49_152
    cfg = N.config(w.vocab, w.eos_id, rows, "bf16", max_tokens=T)
    st = State(cfg, device_table(rows[0], "bf16", 31), device_table(rows[1], "bf16", 32))
    ws = N.Workspace(cfg)
    for win in range(2):
        toks, dys = window_inputs(w, 4 * win, T=T)
        check_window(st, ws, toks, dys, win + 1, w.lr, w.beta2, w.eps, "bf16")
    del st, ws
    torch.cuda.empty_cache()


@pytest.mark.parametrize("T", [1, 64, 65, 127, 128, 129, 4096, 20_000])
def test_single_hot_row(T):
    # every position is the same bigram and trigram (after the first two):
    # one segment spanning up to hundreds of 64-key chunks
    w = workloads.TINY
    N = ng()
    cfg = N.config(w.vocab, w.eos_id, w.rows, "f32", max_tokens=T)
    st = _tiny_state(cfg, w)
    ws = N.Workspace(cfg)
    tok = np.full(T, 42, np.int32)
    toks = [tok] * 4
    dys = [synth.dY(w, 500 + m, T) for m in range(4)]
    check_window(st, ws, toks, dys, 1, w.lr, w.beta2, w.eps, "f32")


def test_spread_equals_burst():
    # The same window in both modes from the same state: each matches the
    # oracle, and the two agree with each other within twice the tolerance.
    w = workloads.SHARD
    N = ng()
    T = 49_152
    base = State(N.config(w.vocab, w.eos_id, w.rows, "bf16", max_tokens=T),
                 device_table(w.rows[0], "bf16", 41), device_table(w.rows[1], "bf16", 42))
    toks, dys = window_inputs(w, 8)
    res = {}
    for m in ("spread", "burst"):
        cfg = N.config(w.vocab, w.eos_id, w.rows, "bf16", max_tokens=T, mode=m)
        st = base.clone()
        st.cfg = cfg
        ws = N.Workspace(cfg)
        rows, grads, orc = check_window(st, ws, toks, dys, 1, w.lr, w.beta2, w.eps, "bf16")
        res[m] = (rows, grads, orc, st)
    for c in range(2):
        rs, Gs, orc, ss = res["spread"][0][c], res["spread"][1][c], res["spread"][2][c], res["spread"][3]
        rb, Gb, sb = res["burst"][0][c], res["burst"][1][c], res["burst"][3]
        np.testing.assert_array_equal(rs, rb)
        helpers.assert_grad_close(Gs, Gb, 2 * orc[2])
        assert torch.equal(ss.tl[c], sb.tl[c])
        idx = torch.from_numpy(rs).cuda()
        Ws = ss.W[c].index_select(0, idx).view(torch.int16).cpu().numpy().view(np.uint16)
        Wb_ = sb.W[c].index_select(0, idx).view(torch.int16).cpu().numpy().view(np.uint16)
        W0 = base.W[c].index_select(0, idx).view(torch.int16).cpu().numpy().view(np.uint16)
        v = sb.v[c].index_select(0, idx).cpu().numpy()
        err, lim = helpers.rows_limit(Ws, Wb_, W0, "bf16", 2 * orc[2], v, w.lr, w.eps)
        assert np.all(err <= 2 * lim)


@pytest.mark.parametrize("mode", ["spread", "burst", "burst_ref"])
def test_bitwise_deterministic(mode):
    w = workloads.SHARD
    N = ng()
    T = 49_152
    cfg = N.config(w.vocab, w.eos_id, w.rows, "bf16", max_tokens=T, mode=mode)
    base = State(cfg, device_table(w.rows[0], "bf16", 51), device_table(w.rows[1], "bf16", 52))
    toks, dys = window_inputs(workloads.COLLISION, 0, T=T)
    res = []
    for rep in range(2):
        st = base.clone()
        ws = N.Workspace(cfg)
        dys_d = [to_dev(dy) for dy in dys]   # burst_ref reads dY at reduce time
        for tok, dy in zip(toks, dys_d):
            N.embed_bwd_accum(cfg, ws, to_dev(tok), dy)
        N.window_reduce(cfg, ws)
        ex = [N.window_export(cfg, ws, c) for c in range(2)]
        st.step(ws, 3, w.lr, w.beta2, w.eps)
        torch.cuda.synchronize()
        del dys_d
        res.append((ex, st))
    for c in range(2):
        assert torch.equal(res[0][0][c][0], res[1][0][c][0])
        assert torch.equal(res[0][0][c][1].view(torch.int32), res[1][0][c][1].view(torch.int32))
        assert torch.equal(res[0][1].W[c].view(torch.int16), res[1][1].W[c].view(torch.int16))
        assert torch.equal(res[0][1].v[c].view(torch.int32), res[1][1].v[c].view(torch.int32))


def test_empty_window_step_is_noop():
    w = workloads.TINY
    N = ng()
    cfg = N.config(w.vocab, w.eos_id, w.rows, "f32", max_tokens=64)
    st = _tiny_state(cfg, w)
    before = st.clone()
    ws = N.Workspace(cfg)
    N.embed_bwd_accum(cfg, ws, torch.zeros(0, dtype=torch.int32, device="cuda"),
                      torch.zeros((0, 768), device="cuda"))
    st.step(ws, 1, 0.01, 0.95, 1e-8)
    for c in range(2):
        assert torch.equal(st.W[c], before.W[c])
        assert torch.equal(st.v[c], before.v[c])
        assert torch.equal(st.tl[c], before.tl[c])
    assert N.device_status(cfg, ws) == 0


def test_window_full_flag():
    w = workloads.TINY
    N = ng()
    cfg = N.config(w.vocab, w.eos_id, w.rows, "f32", max_tokens=2048, window_rows=100)
    st = _tiny_state(cfg, w)
    ws = N.Workspace(cfg)
    tok = synth.tokens(w, 0)
    N.embed_bwd_accum(cfg, ws, to_dev(tok), to_dev(synth.dY(w, 0)))
    rows, G = N.window_export(cfg, ws, 0)
    assert len(rows) == 100
    st.step(ws, 1, 0.01, 0.95, 1e-8)
    assert N.device_status(cfg, ws, clear=True) & N.FLAG_WINDOW_FULL
    assert int((st.tl[0] == 1).sum()) == 100


def test_stash_full_flag_burst():
    w = workloads.TINY
    N = ng()
    cfg = N.config(w.vocab, w.eos_id, w.rows, "f32", max_tokens=256, accum_steps=2, mode="burst")
    ws = N.Workspace(cfg)
    for s in range(3):   # one micro-step more than the window holds
        N.embed_bwd_accum(cfg, ws, to_dev(synth.tokens(w, s, 256)), to_dev(synth.dY(w, s, 256)))
    assert N.device_status(cfg, ws, clear=True) & N.FLAG_STASH_FULL


def test_step_order_flag():
    w = workloads.TINY
    N = ng()
    cfg = N.config(w.vocab, w.eos_id, w.rows, "f32", max_tokens=64)
    st = _tiny_state(cfg, w)
    ws = N.Workspace(cfg)
    for t in (5, 5):   # the second step does not advance t
        N.embed_bwd_accum(cfg, ws, to_dev(synth.tokens(w, 0, 64)), to_dev(synth.dY(w, 0, 64)))
        st.step(ws, t, 0.01, 0.95, 1e-8)
    assert N.device_status(cfg, ws, clear=True) & N.FLAG_STEP_ORDER


@pytest.mark.parametrize("how", ["export", "step", "fused_last"])
@pytest.mark.parametrize("mode", ["spread", "burst", "burst_ref"])
def test_tiny_workload_bf16_dy(mode, how):
    # bf16 upstream gradients (the gradient of a bf16 forward output): the
    # kernels widen each element exactly and sum in fp32, so the oracle gets
    # the same values as float32
    w = workloads.TINY
    N = ng()
    cfg = N.config(w.vocab, w.eos_id, w.rows, "f32", max_tokens=w.tokens_per_step, mode=mode,
                   dy_dtype="bf16")
    st = _tiny_state(cfg, w)
    ws = N.Workspace(cfg)
    for win in range(w.steps // w.accum_steps):
        toks, dys = window_inputs(w, win * w.accum_steps)
        dys = [round_to_bf16(d) for d in dys]
        check_window(st, ws, toks, dys, win + 1, w.lr, w.beta2, w.eps, "f32", how=how, dy_dtype="bf16")
    assert N.device_status(cfg, ws) == 0


@pytest.mark.parametrize("mode,how", [("spread", "fused_last"), ("burst", "step"), ("burst_ref", "step"),
                                      ("burst_ref", "fused_last")])
def test_shard_workload_bf16_dy(mode, how):
    w = workloads.COLLISION
    N = ng()
    rows = workloads.SHARD.rows
    T = 49_152
    cfg = N.config(w.vocab, w.eos_id, rows, "bf16", max_tokens=T, mode=mode, dy_dtype="bf16")
    st = State(cfg, device_table(rows[0], "bf16", 71), device_table(rows[1], "bf16", 72))
    ws = N.Workspace(cfg)
    for win in range(2):
        toks, dys = window_inputs(w, 4 * win, T=T)
        dys = [round_to_bf16(d) for d in dys]
        check_window(st, ws, toks, dys, win + 1, w.lr, w.beta2, w.eps, "bf16", how=how, dy_dtype="bf16")
    assert N.device_status(cfg, ws) == 0
    del st, ws
    torch.cuda.empty_cache()


def test_bf16_dy_matches_f32_dy_bitwise():
    # the same bf16-valued gradients given as fp32 or as bf16 take the same
    # path through the same sums: the results are bitwise equal
    w = workloads.TINY
    N = ng()
    outs = []
    for dyt in ("f32", "bf16"):
        cfg = N.config(w.vocab, w.eos_id, w.rows, "f32", max_tokens=w.tokens_per_step, mode="burst_ref",
                       dy_dtype=dyt)
        st = _tiny_state(cfg, w)
        ws = N.Workspace(cfg)
        toks, dys = window_inputs(w, 0)
        keep = [to_dev(round_to_bf16(d)) for d in dys]
        if dyt == "bf16":
            keep = [k.to(torch.bfloat16) for k in keep]
        for tok, dy in zip(toks, keep):
            N.embed_bwd_accum(cfg, ws, to_dev(tok), dy)
        st.step(ws, 1, w.lr, w.beta2, w.eps)
        torch.cuda.synchronize()
        outs.append((st.W[0].cpu(), st.W[1].cpu(), st.st[0].cpu(), st.st[1].cpu()))
    for a, b in zip(*outs):
        assert torch.equal(a, b)


@pytest.mark.parametrize("mode", ["burst", "burst_ref"])
def test_radix_tile_size_does_not_change_results(mode):
    # burst windows sort 4 x max_tokens keys per channel: from 2^20 keys on
    # the radix kernels take 4,096-key tiles, below it 2,048-key tiles.  The
    # sort is stable either way, so a ragged window stepped through both
    # configurations must give the same bits (both with the nested sort,
    # which windows below 2^20 keys take only when asked to).
    N = ng()
    w = workloads.FULL
    rows = (1 << 20, 1 << 20)
    Ts = [262143, 100000, 7, 150001]
    inputs = [[(to_dev(synth.tokens(w, 700 + 4 * win + m, T)), to_dev(synth.dY(w, 700 + 4 * win + m, T)))
               for m, T in enumerate(Ts)] for win in range(2)]
    states = []
    for max_tokens in (262144, 262143):   # 4 x 262,144 = 2^20 keys; 4 x 262,143 just below
        cfg = N.config(w.vocab, w.eos_id, rows, "bf16", max_tokens=max_tokens, mode=mode, nest_always=True)
        st = State(cfg, device_table(rows[0], "bf16", 41), device_table(rows[1], "bf16", 42))
        ws = N.Workspace(cfg)
        for win in range(2):
            for m, (tok, dy) in enumerate(inputs[win]):
                if m == len(Ts) - 1:
                    st.bwd_step(ws, tok, dy, win + 1, w.lr, w.beta2, w.eps)
                else:
                    N.embed_bwd_accum(cfg, ws, tok, dy)
        torch.cuda.synchronize()
        assert N.device_status(cfg, ws) == 0
        assert int((st.tl[0] == 2).sum()) > 0
        states.append(st)
        del ws
    for c in range(2):
        assert torch.equal(states[0].W[c], states[1].W[c]), c
        assert torch.equal(states[0].st[c], states[1].st[c]), c
