"""GPU-side helpers shared by the GPU tests (tables, state snapshots, a window
driver that checks every step against the oracle).  Test infrastructure."""
from __future__ import annotations

import numpy as np
import torch

import helpers
import oracle
from sparse_hashed_gram_amd import synth


def ng():
    from sparse_hashed_gram_amd import ngram
    return ngram


def device_table(R: int, dtype: str, seed: int, chunk: int = 1 << 20) -> torch.Tensor:
    """N(0, 0.02) table generated on the device in row chunks."""
    tdt = torch.float32 if dtype == "f32" else torch.bfloat16
    W = torch.empty((R, 768), dtype=tdt, device="cuda")
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    for s in range(0, R, chunk):
        e = min(R, s + chunk)
        W[s:e] = (torch.randn((e - s, 768), generator=g, device="cuda") * 0.02).to(tdt)
    return W


def host_rows(W: torch.Tensor, rows: np.ndarray) -> np.ndarray:
    """Rows of a device table as numpy (float32, or uint16 bf16 bits)."""
    idx = torch.from_numpy(np.ascontiguousarray(rows, np.int64)).cuda()
    x = W.index_select(0, idx)
    if x.dtype == torch.bfloat16:
        return x.view(torch.int16).cpu().numpy().view(np.uint16)
    return x.cpu().numpy()


def host_vec(x: torch.Tensor, rows: np.ndarray) -> np.ndarray:
    idx = torch.from_numpy(np.ascontiguousarray(rows, np.int64)).cuda()
    return x.index_select(0, idx).cpu().numpy()


class State:
    """Tables and optimizer state (packed v, t_last records) of both channels."""

    def __init__(self, cfg, W_b, W_t):
        self.cfg = cfg
        self.W = [W_b, W_t]
        self.st = [ng().new_state(cfg.rows[c]) for c in range(2)]

    @property
    def v(self):
        return [ng().state_v(x) for x in self.st]

    @property
    def tl(self):
        return [ng().state_t_last(x) for x in self.st]

    def clone(self):
        s = State(self.cfg, self.W[0].clone(), self.W[1].clone())
        s.st = [x.clone() for x in self.st]
        return s

    def step(self, ws, t, lr, beta2, eps):
        ng().sparse_step(self.cfg, ws, self.W[0], self.W[1], self.st[0], self.st[1], t, lr, beta2, eps)

    def bwd_step(self, ws, tok, dy, t, lr, beta2, eps):
        ng().embed_bwd_step(self.cfg, ws, tok, dy, self.W[0], self.W[1], self.st[0], self.st[1], t, lr,
                            beta2, eps)


def to_dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def dy_dev(dy: np.ndarray, dy_dtype: str = "f32") -> torch.Tensor:
    """dY on the device in the config's dY dtype.  For bf16 the float32
    values must already be bf16 numbers (round_to_bf16), so the upload is exact
    and the oracle sees the same gradients."""
    t = to_dev(dy)
    if dy_dtype == "f32":
        return t
    b = t.to(torch.bfloat16)
    same = torch.isclose(b.to(torch.float32), t, rtol=0.0, atol=0.0, equal_nan=True)
    assert bool(same.all()), "dY is not made of bf16 values"
    return b


def round_to_bf16(dy: np.ndarray) -> np.ndarray:
    """float32 array of the nearest bf16 numbers (test input preparation)."""
    return torch.from_numpy(np.ascontiguousarray(dy)).to(torch.bfloat16).to(torch.float32).numpy()


def check_window(st: State, ws, toks, dys, t, lr, beta2, eps, dtype, seeds=(1, 2),
                 sample_untouched=512, keep_rows=None, rng_seed=0, how="export", dy_dtype="f32"):
    """Feeds one window (lists of numpy tokens / dY) through the GPU path,
    checks the touched sets and the step against the oracle, and a sample of
    untouched rows for bitwise stability.  how:
      "export"     reduce, export and check the window gradient, then step;
      "step"       sparse_step straight after the micro-steps (burst mode:
                   the reduction fused with the step);
      "fused_last" the last micro-step through embed_bwd_step."""
    N = ng()
    cfg = st.cfg
    last = len(toks) - 1 if how == "fused_last" else len(toks)
    keep = []   # burst by reference reads dY at step time: keep it alive
    for tok, dy in zip(toks[:last], dys[:last]):
        keep.append(dy_dev(dy, dy_dtype))
        N.embed_bwd_accum(cfg, ws, to_dev(tok), keep[-1])
    if how == "export":
        N.window_reduce(cfg, ws)
    orc = helpers.oracle_window(cfg.vocab, cfg.eos_id, (cfg.rows[0], cfg.rows[1]), toks, dys,
                                seeds, keep_rows=keep_rows)
    if how != "export":
        return _check_step_only(st, ws, toks, dys, t, lr, beta2, eps, dtype, orc, how, last,
                                sample_untouched, rng_seed, keep, dy_dtype)
    rs = np.random.default_rng(rng_seed)
    touched_all = []
    grads = []
    snaps = []
    for c in range(2):
        rows_g, G_g = N.window_export(cfg, ws, c)
        rows_g = rows_g.cpu().numpy()
        G_g = G_g.cpu().numpy()
        assert len(np.unique(rows_g)) == len(rows_g), "duplicate rows in the window"
        order = np.argsort(rows_g, kind="stable")
        rows_g, G_g = rows_g[order], G_g[order]
        touched, G_o, A_o = orc[c]
        if keep_rows is None:
            np.testing.assert_array_equal(rows_g, touched)
            G_cmp = G_g
        else:
            # the oracle saw only the sampled rows: they must all be touched
            pos = np.searchsorted(rows_g, touched)
            assert np.all(pos < len(rows_g)) and np.array_equal(rows_g[pos], touched)
            G_cmp = G_g[pos]
        helpers.assert_grad_close(G_cmp, G_o, A_o)
        touched_all.append(rows_g)
        grads.append(G_g)
        # state snapshot of the rows the oracle will step
        Wb = host_rows(st.W[c], touched)
        vb = host_vec(st.v[c], touched)
        tb = host_vec(st.tl[c], touched)
        # untouched sample
        cand = rs.integers(0, cfg.rows[c], size=4 * sample_untouched)
        cand = np.setdiff1d(cand, rows_g)[:sample_untouched]
        snaps.append((touched, G_o, A_o, Wb, vb, tb, cand, host_rows(st.W[c], cand),
                      host_vec(st.v[c], cand), host_vec(st.tl[c], cand)))
    st.step(ws, t, lr, beta2, eps)
    del keep
    for c in range(2):
        touched, G_o, A_o, Wb, vb, tb, cand, Wc, vc, tc = snaps[c]
        W_o, v_o, t_o = oracle.sparse_step(G_o, Wb, vb, tb, t, lr, beta2, eps)
        W_g = host_rows(st.W[c], touched)
        v_g = host_vec(st.v[c], touched)
        t_g = host_vec(st.tl[c], touched)
        np.testing.assert_array_equal(t_g, t_o)
        helpers.assert_v_close(v_g, v_o, G=G_o, absbound=A_o, beta2=beta2)
        helpers.assert_rows_close(W_g, W_o, Wb, dtype, G=G_o, absbound=A_o, v_orc=v_o, lr=lr,
                                  eps=eps)
        np.testing.assert_array_equal(host_rows(st.W[c], cand), Wc)
        np.testing.assert_array_equal(host_vec(st.v[c], cand), vc)
        np.testing.assert_array_equal(host_vec(st.tl[c], cand), tc)
    # the window is empty afterwards
    for c in range(2):
        r, _ = N.window_export(cfg, ws, c, with_grad=False)
        assert len(r) == 0
    return touched_all, grads, orc


def window_inputs(w, first_step, T=None, n=4, tok_fn=None):
    toks, dys = [], []
    for s in range(first_step, first_step + n):
        toks.append(synth.tokens(w, s, T) if tok_fn is None else tok_fn(s))
        dys.append(synth.dY(w, s, len(toks[-1])))
    return toks, dys


def oracle_snapshots(st: State, orc, rs, sample_untouched=512):
    """Pre-step state of the rows the oracle will step (per channel: the
    oracle's touched rows, G and sum |s dY|, their W, v, t_last) and of a
    sample of untouched rows.  Take it before the window's step."""
    snaps = []
    for c in range(2):
        touched, G_o, A_o = orc[c]
        cand = rs.integers(0, st.cfg.rows[c], size=4 * sample_untouched)
        cand = np.setdiff1d(cand, touched)[:sample_untouched]
        snaps.append(dict(touched=touched, G=G_o, A=A_o, W=host_rows(st.W[c], touched),
                          v=host_vec(st.v[c], touched), tl=host_vec(st.tl[c], touched), cand=cand,
                          Wc=host_rows(st.W[c], cand), vc=host_vec(st.v[c], cand),
                          tc=host_vec(st.tl[c], cand)))
    return snaps


def check_step_against_oracle(st: State, snaps, t, lr, beta2, eps, dtype, skip=None):
    """After the window's step: t_last of every touched row exact (and no
    other row at t), v and W of the touched rows within tolerance of the
    oracle's step from the snapshot, untouched samples bitwise unchanged.
    skip[c]: rows left out of the tolerance checks (the caller checks them
    itself).  Returns the oracle's (W, v) per channel."""
    torch.cuda.synchronize()
    res = []
    for c in range(2):
        s = snaps[c]
        touched = s["touched"]
        W_o, v_o, t_o = oracle.sparse_step(s["G"], s["W"], s["v"], s["tl"], t, lr, beta2, eps)
        np.testing.assert_array_equal(host_vec(st.tl[c], touched), t_o)
        assert int((st.tl[c] == t).sum()) == len(touched)
        keep = np.ones(len(touched), bool) if skip is None else ~np.isin(touched, skip[c])
        rows = touched[keep]
        helpers.assert_v_close(host_vec(st.v[c], rows), v_o[keep], G=s["G"][keep], absbound=s["A"][keep],
                               beta2=beta2)
        helpers.assert_rows_close(host_rows(st.W[c], rows), W_o[keep], s["W"][keep], dtype, G=s["G"][keep],
                                  absbound=s["A"][keep], v_orc=v_o[keep], lr=lr, eps=eps)
        np.testing.assert_array_equal(host_rows(st.W[c], s["cand"]), s["Wc"])
        np.testing.assert_array_equal(host_vec(st.v[c], s["cand"]), s["vc"])
        np.testing.assert_array_equal(host_vec(st.tl[c], s["cand"]), s["tc"])
        res.append((W_o, v_o))
    return res


def window_oracle(cfg, toks, dys, seeds=(1, 2)):
    """The oracle's window gradient per channel for numpy token / dY lists."""
    return helpers.oracle_window(cfg.vocab, cfg.eos_id, (cfg.rows[0], cfg.rows[1]), toks, dys, seeds)


def _check_step_only(st, ws, toks, dys, t, lr, beta2, eps, dtype, orc, how, last, sample_untouched,
                     rng_seed, keep, dy_dtype="f32"):
    """check_window without the exported gradient: the step's results alone."""
    N = ng()
    cfg = st.cfg
    snaps = oracle_snapshots(st, orc, np.random.default_rng(rng_seed), sample_untouched)
    if how == "fused_last":
        st.bwd_step(ws, to_dev(toks[last]), dy_dev(dys[last], dy_dtype), t, lr, beta2, eps)
    else:
        st.step(ws, t, lr, beta2, eps)
    torch.cuda.synchronize()
    keep.clear()
    check_step_against_oracle(st, snaps, t, lr, beta2, eps, dtype)
    for c in range(2):
        r, _ = N.window_export(cfg, ws, c, with_grad=False)
        assert len(r) == 0
    return [s["touched"] for s in snaps], None, orc
