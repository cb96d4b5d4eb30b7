"""The allocation-free window step against the regular entry points.

ngram_window_step_noalloc runs a whole accumulation window with the
library's fixed device array as its workspace.  It must give bitwise the
results of the regular calls on a fresh workspace of the same burst-by-
reference configuration (ngram_embed_bwd_accum for the first micro-steps,
ngram_embed_bwd_step for the last): the same kernels on the same inputs.
Two calls in a row, the second on a smaller window, so the second finds the
first one's contents in the array; each window is also checked against the
oracle.
"""
import numpy as np
import pytest
import torch

from gpu_common import State, check_step_against_oracle, ng, oracle_snapshots, to_dev, window_oracle
from sparse_hashed_gram_amd import synth, workloads

pytestmark = pytest.mark.gpu

W = workloads.TINY


def _regular(N, cfg0, st, toks, dys, n, T, t):
    cfg = N.config(cfg0.vocab, cfg0.eos_id, (cfg0.rows[0], cfg0.rows[1]),
                   "f32" if cfg0.dtype == N.DTYPE_F32 else "bf16", max_tokens=T, accum_steps=n,
                   mode="burst_ref", nest_always=bool(cfg0.options & N.OPT_NEST_ALWAYS))
    ws = N.Workspace(cfg)
    for m in range(n - 1):
        N.embed_bwd_accum(cfg, ws, toks[m], dys[m])
    N.embed_bwd_step(cfg, ws, toks[n - 1], dys[n - 1], st.W[0], st.W[1], st.st[0], st.st[1], t, W.lr, W.beta2,
                     W.eps)
    torch.cuda.synchronize()
    assert N.device_status(cfg, ws) == 0


@pytest.mark.parametrize("nest", [False, True])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_noalloc_window_equals_the_regular_path(dtype, nest):
    # nest: the nested sort and its run pieces in the fixed array too
    N = ng()
    cfg = N.config(W.vocab, W.eos_id, W.rows, dtype, max_tokens=2048, nest_always=nest)   # mode etc. are not used
    tdt = torch.float32 if dtype == "f32" else torch.bfloat16
    reg = State(cfg, to_dev(synth.init_rows(W, 0, W.rows[0])).to(tdt),
                to_dev(synth.init_rows(W, 1, W.rows[1])).to(tdt))
    nal = reg.clone()
    flags = torch.zeros(1, dtype=torch.int32, device="cuda")
    for call, (n, T) in enumerate([(4, 2048), (3, 700)]):
        toks_np = [synth.tokens(W, 10 * call + m, T) for m in range(n)]
        dys_np = [synth.dY(W, 10 * call + m, T) for m in range(n)]
        toks = [to_dev(x) for x in toks_np]
        dys = [to_dev(x) for x in dys_np]
        t = call + 1
        snaps = oracle_snapshots(nal, window_oracle(cfg, toks_np, dys_np), np.random.default_rng(call))
        _regular(N, cfg, reg, toks, dys, n, T, t)
        N.window_step_noalloc(cfg, torch.cat(toks), torch.cat(dys), T, n, nal.W[0], nal.W[1], nal.st[0],
                              nal.st[1], t, W.lr, W.beta2, W.eps, flags=flags)
        torch.cuda.synchronize()
        for c in range(2):
            assert torch.equal(reg.W[c], nal.W[c]), (call, c)
            assert torch.equal(reg.st[c], nal.st[c]), (call, c)
        check_step_against_oracle(nal, snaps, t, W.lr, W.beta2, W.eps, dtype)
    assert int(flags.item()) == 0


def test_noalloc_flags_bad_tokens():
    N = ng()
    cfg = N.config(W.vocab, W.eos_id, W.rows, "f32", max_tokens=256)
    st = State(cfg, to_dev(synth.init_rows(W, 0, W.rows[0])), to_dev(synth.init_rows(W, 1, W.rows[1])))
    tok = synth.tokens(W, 3, 256)
    tok[7] = W.vocab + 5
    flags = torch.zeros(1, dtype=torch.int32, device="cuda")
    N.window_step_noalloc(cfg, to_dev(tok), to_dev(synth.dY(W, 3, 256)), 256, 1, st.W[0], st.W[1], st.st[0],
                          st.st[1], 1, W.lr, W.beta2, W.eps, flags=flags)
    torch.cuda.synchronize()
    assert int(flags.item()) & N.FLAG_BAD_TOKEN
