"""GPU parity at full size: the 84.6M-row bf16 table (2 x 42,300,000 x 768,
about 130 GB) on one GPU, 393,216 tokens per micro-step, the launch
configuration bench.py times.  The oracle cannot hold the whole table, so
outputs are checked on samples it computes one by one:

- forward: 4,096 sampled positions per micro-step, bit-exact;
- the window's touched rows in ascending order (ngram_touched_rows), exact;
- backward: the full touched set (exact), and the window gradient of sampled
  rows (random touched rows plus the hottest ones), fed to the oracle with
  exactly the entries hashed to those rows;
- step: the sampled rows' W, v, t_last against the oracle's step from the
  GPU's pre-step state, every touched row's t_last, untouched samples bitwise
  unchanged;
- spread, copying burst and burst by reference (fused entry point) over 8
  windows = 32 steps from the same state (restoring the touched rows between
  the runs), each against the oracle and the bursts against spread on every
  touched row;
- bf16 upstream gradients in the launch sequence bench.py --dy-dtype bf16
  times (burst by reference, the window reduced fused with the step).
"""
import numpy as np
import pytest
import torch

import helpers
import oracle
from gpu_common import host_rows, host_vec, ng, to_dev
from sparse_hashed_gram_amd import synth, workloads

pytestmark = [pytest.mark.gpu, pytest.mark.big]

FULL = workloads.FULL
T = FULL.tokens_per_step


def _free_gib():
    free, _ = torch.cuda.mem_get_info()
    return free / 2**30


@pytest.fixture(scope="module")
def big_state():
    torch.cuda.empty_cache()
    if _free_gib() < 200:
        pytest.skip("needs about 200 GiB of free device memory")
    N = ng()
    cfg = N.config(FULL.vocab, FULL.eos_id, FULL.rows, "bf16", max_tokens=T)
    W = []
    for c in range(2):
        t = torch.empty((FULL.rows[c], 768), dtype=torch.bfloat16, device="cuda")
        g = torch.Generator(device="cuda")
        g.manual_seed(900 + c)
        for s in range(0, FULL.rows[c], 1 << 21):
            e = min(FULL.rows[c], s + (1 << 21))
            t[s:e] = (torch.randn((e - s, 768), generator=g, device="cuda") * 0.02).to(torch.bfloat16)
        W.append(t)
    state = [N.new_state(FULL.rows[c]) for c in range(2)]
    st = {"cfg": cfg, "W": W, "state": state,
          "v": [N.state_v(x) for x in state], "tl": [N.state_t_last(x) for x in state], "t": 0}
    yield st
    del st
    torch.cuda.empty_cache()


def _dy(seed):
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    return torch.randn((T, 768), generator=g, device="cuda")


def _sample_rows(rows_all, rs, n_rand=1500, n_hot=24):
    """Random touched rows plus the most frequent ones."""
    u, cnt = np.unique(rows_all, return_counts=True)
    hot = u[np.argsort(-cnt)[:n_hot]]
    rnd = rs.choice(u, size=min(n_rand, len(u)), replace=False)
    return np.unique(np.concatenate([hot, rnd])), int(cnt.max())


def _oracle_grad_for(rows_all, neg_all, dys, sample):
    """Oracle window gradient of the sampled rows only (every entry hashed to
    them, in stream order).  dY rows are fetched from the device."""
    m = np.isin(rows_all, sample)
    pos = np.flatnonzero(m)
    step_of = pos // T
    dY = np.empty((len(pos), 768), np.float32)
    for s in range(len(dys)):
        sel = step_of == s
        if sel.any():
            idx = torch.from_numpy(pos[sel] - s * T).cuda()
            dY[sel] = dys[s].index_select(0, idx).float().cpu().numpy()   # bf16 widens exactly
    touched, G = oracle.window_grad(rows_all[m], neg_all[m], dY)
    _, A = oracle.window_grad(rows_all[m], np.zeros(len(pos), np.uint8), np.abs(dY))
    return touched, G, A


def _run_and_check_window(st, ws, toks, dy_seeds, rs, check_fwd=True, fused_last=False, dy_dtype="f32"):
    """One window through the GPU path, checked on sampled rows.  fused_last:
    the last micro-step goes through ngram_embed_bwd_step (the reduction
    fused with the step), so the window gradient is only seen through the
    step's results."""
    N = ng()
    cfg = st["cfg"]
    dys = [_dy(s) if dy_dtype == "f32" else _dy(s).to(torch.bfloat16) for s in dy_seeds]
    per = [helpers.oracle_rows(FULL, tok, FULL.rows) for tok in toks]
    out = torch.empty((T, 768), dtype=torch.bfloat16, device="cuda")
    for m, tok in enumerate(toks):
        tok_d = to_dev(tok)
        if check_fwd:
            N.embed_fwd(cfg, st["W"][0], st["W"][1], tok_d, out=out)
            sp = np.sort(rs.choice(T, size=4096, replace=False))
            sp[:3] = [0, 1, 2]   # the context-start positions
            rb, nb, rt, nt = (x[sp] for x in per[m])
            ib, it = np.unique(rb), np.unique(rt)
            ref = oracle.forward(host_rows(st["W"][0], ib), host_rows(st["W"][1], it), rb, nb, rt, nt,
                                 ids_b=ib, ids_t=it, out_dtype="bf16")
            got = out.index_select(0, torch.from_numpy(sp).cuda()).view(torch.int16).cpu().numpy()
            np.testing.assert_array_equal(got.view(np.uint16), ref)
        if fused_last and m == len(toks) - 1:
            last_tok = tok_d
            break
        N.embed_bwd_accum(cfg, ws, tok_d, dys[m])
    if not fused_last:
        # the window's distinct rows, ascending, before any reduce in the
        # burst modes (read from the stash) or after the spread reduces
        for c in range(2):
            got, cnt = N.touched_rows(cfg, ws, c)
            want = np.unique(np.concatenate([p[2 * c] for p in per]))
            assert int(cnt.item()) == len(want)
            np.testing.assert_array_equal(got[:len(want)].cpu().numpy().astype(np.int64), want)
            del got
        N.window_reduce(cfg, ws)
    snaps = []
    for c in range(2):
        rows_all = np.concatenate([p[2 * c] for p in per])
        neg_all = np.concatenate([p[2 * c + 1] for p in per])
        sample, hottest = _sample_rows(rows_all, rs)
        touched, G_o, A_o = _oracle_grad_for(rows_all, neg_all, dys, sample)
        assert np.array_equal(touched, sample)
        if fused_last:
            rows_g = torch.from_numpy(np.unique(rows_all)).cuda()
        else:
            rows_g, G_g = N.window_export(cfg, ws, c)
            order = torch.argsort(rows_g)
            rows_g, G_g = rows_g[order], G_g[order]
            np.testing.assert_array_equal(rows_g.cpu().numpy(), np.unique(rows_all))
            pos = torch.searchsorted(rows_g, torch.from_numpy(sample).cuda())
            helpers.assert_grad_close(G_g.index_select(0, pos).cpu().numpy(), G_o, A_o)
            del G_g
        cand = rs.integers(0, FULL.rows[c], size=4096)
        cand = np.setdiff1d(cand, rows_g.cpu().numpy())[:1024]
        snaps.append(dict(sample=sample, G=G_o, A=A_o, hottest=hottest, rows_g=rows_g,
                          W=host_rows(st["W"][c], sample), v=host_vec(st["v"][c], sample),
                          tl=host_vec(st["tl"][c], sample), cand=cand,
                          Wc=host_rows(st["W"][c], cand)))
    st["t"] += 1
    t = st["t"]
    if fused_last:
        N.embed_bwd_step(cfg, ws, last_tok, dys[-1], st["W"][0], st["W"][1], st["state"][0],
                         st["state"][1], t, FULL.lr, FULL.beta2, FULL.eps)
    else:
        N.sparse_step(cfg, ws, st["W"][0], st["W"][1], st["state"][0], st["state"][1], t, FULL.lr,
                      FULL.beta2, FULL.eps)
    for c in range(2):
        s = snaps[c]
        W_o, v_o, t_o = oracle.sparse_step(s["G"], s["W"], s["v"], s["tl"], t, FULL.lr, FULL.beta2,
                                           FULL.eps)
        np.testing.assert_array_equal(host_vec(st["tl"][c], s["sample"]), t_o)
        helpers.assert_v_close(host_vec(st["v"][c], s["sample"]), v_o, G=s["G"], absbound=s["A"],
                               beta2=FULL.beta2)
        helpers.assert_rows_close(host_rows(st["W"][c], s["sample"]), W_o, s["W"], "bf16")
        assert int((st["tl"][c] == t).sum()) == len(s["rows_g"])
        assert bool((st["tl"][c].index_select(0, s["rows_g"]) == t).all())
        np.testing.assert_array_equal(host_rows(st["W"][c], s["cand"]), s["Wc"])
    for c in range(2):   # the window is empty after the step
        assert len(N.window_export(cfg, ws, c, with_grad=False)[0]) == 0
    assert N.device_status(cfg, ws) == 0
    return snaps


def test_full_table_window_spread(big_state):
    N = ng()
    ws = N.Workspace(big_state["cfg"])
    rs = np.random.default_rng(3)
    toks = [synth.tokens(FULL, s) for s in range(4)]
    snaps = _run_and_check_window(big_state, ws, toks, [31, 32, 33, 34], rs)
    assert snaps[0]["hottest"] > 10_000   # hot bigram segments span hundreds of chunks


def test_full_table_window_fused_step(big_state):
    # the launch sequence bench.py times: three micro-steps accumulated, the
    # last one reduced together with the sparse step
    N = ng()
    ws = N.Workspace(big_state["cfg"])
    rs = np.random.default_rng(6)
    for win in range(2):
        toks = [synth.tokens(FULL, 40 + 4 * win + m) for m in range(4)]
        snaps = _run_and_check_window(big_state, ws, toks, [61 + 4 * win + m for m in range(4)], rs,
                                      check_fwd=win == 0, fused_last=True)
        assert snaps[0]["hottest"] > 10_000


def test_collision_workload_full_table(big_state):
    N = ng()
    w = workloads.COLLISION
    ws = N.Workspace(big_state["cfg"])
    rs = np.random.default_rng(4)
    toks = [synth.tokens(w, s) for s in range(4)]
    snaps = _run_and_check_window(big_state, ws, toks, [41, 42, 43, 44], rs, check_fwd=False)
    assert snaps[0]["hottest"] > 50_000


def test_spread_vs_burst_full_table(big_state):
    """The spread-vs-burst workload, 32 steps = 8 windows: each window runs in
    spread mode (micro-steps reduced as they come, then the step), in copying
    burst mode, and in burst-by-reference mode through the fused entry point,
    each from the same state; each is checked against the oracle on sampled
    rows, and both burst runs are compared with the spread run on every
    touched row."""
    N = ng()
    w = workloads.SPREAD_BURST
    cfg_s = big_state["cfg"]
    cfgs = {"burst": N.config(w.vocab, w.eos_id, w.rows, "bf16", max_tokens=T, mode="burst"),
            "burst_ref": N.config(w.vocab, w.eos_id, w.rows, "bf16", max_tokens=T, mode="burst_ref")}
    ws_s = N.Workspace(cfg_s)
    wss = {m: N.Workspace(c) for m, c in cfgs.items()}
    rs = np.random.default_rng(5)
    for win in range(8):
        toks = [synth.tokens(w, 4 * win + m) for m in range(4)]
        seeds = [500 + 4 * win + m for m in range(4)]
        idx = [[N.hash(cfg_s, to_dev(tok))[c] & 0x7FFFFFFF for tok in toks] for c in range(2)]
        rows = [torch.unique(torch.cat(idx[c]).long()) for c in range(2)]
        keep = [(big_state["W"][c].index_select(0, rows[c]),
                 big_state["state"][c].index_select(0, rows[c])) for c in range(2)]
        t0 = big_state["t"]
        big_state["cfg"] = cfg_s
        _run_and_check_window(big_state, ws_s, toks, seeds, rs, check_fwd=False)
        spread = [(big_state["W"][c].index_select(0, rows[c]), big_state["v"][c].index_select(0, rows[c]))
                  for c in range(2)]
        for mode in ("burst", "burst_ref"):
            for c in range(2):   # restore the touched rows: the state is as before the window
                big_state["W"][c].index_copy_(0, rows[c], keep[c][0])
                big_state["state"][c].index_copy_(0, rows[c], keep[c][1])
            big_state["t"] = t0
            big_state["cfg"] = cfgs[mode]
            _run_and_check_window(big_state, wss[mode], toks, seeds, rs, check_fwd=False,
                                  fused_last=mode == "burst_ref")
            big_state["cfg"] = cfg_s
            for c in range(2):
                Wb = big_state["W"][c].index_select(0, rows[c])
                vb = big_state["v"][c].index_select(0, rows[c])
                Ws, vs = spread[c]
                # every touched row: bf16 values within 2 ulp + a small absolute
                # floor for cancellations (the sampled rows are held to the full
                # oracle tolerance above)
                a, b = Ws.float(), Wb.float()
                ulp = torch.maximum(a.abs(), b.abs()) * 2.0 ** -7
                upd = (b - keep[c][0].float()).abs()
                assert bool(((a - b).abs() <= 2 * ulp + 2e-5 * upd + 1e-5).all()), (win, mode, c)
                assert bool(((vs - vb).abs() <= 1e-3 * vb.abs() + 1e-12).all()), (win, mode, c)


def test_full_table_bf16_dy_burst_ref(big_state):
    N = ng()
    cfg = N.config(FULL.vocab, FULL.eos_id, FULL.rows, "bf16", max_tokens=T, mode="burst_ref",
                   dy_dtype="bf16")
    ws = N.Workspace(cfg)
    rs = np.random.default_rng(8)
    saved = big_state["cfg"]
    big_state["cfg"] = cfg
    try:
        for win in range(2):
            toks = [synth.tokens(FULL, 80 + 4 * win + m) for m in range(4)]
            snaps = _run_and_check_window(big_state, ws, toks, [81 + 4 * win + m for m in range(4)], rs,
                                          check_fwd=False, fused_last=True, dy_dtype="bf16")
            assert snaps[0]["hottest"] > 10_000
    finally:
        big_state["cfg"] = saved
