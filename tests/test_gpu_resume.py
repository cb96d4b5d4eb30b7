"""Resuming at a window boundary gives bitwise the same run.

With beta2 applied retroactively (the @classiclarryd post quoted on the
airebao.com item), a row's pending decay is implied by t - t_last, so the
tables, each row's (v, t_last) record and the next step number are the
whole optimizer state between windows.  A run saved after its second window,
restored into new tensors and a new workspace, and continued for two more
windows must end bitwise equal to the same four windows run without a break.
"""
import numpy as np
import pytest
import torch

from gpu_common import State, ng, to_dev, window_inputs
from sparse_hashed_gram_amd import synth, workloads

pytestmark = pytest.mark.gpu

W = workloads.TINY


def _window(N, cfg, st, ws, toks, dys, t):
    for m in range(len(toks) - 1):
        N.embed_bwd_accum(cfg, ws, toks[m], dys[m])
    st.bwd_step(ws, toks[-1], dys[-1], t, W.lr, W.beta2, W.eps)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("mode", ["spread", "burst", "burst_ref"])
def test_resume_at_window_boundary_is_bitwise(mode, dtype):
    N = ng()
    cfg = N.config(W.vocab, W.eos_id, W.rows, dtype, max_tokens=W.tokens_per_step, mode=mode)
    tdt = torch.float32 if dtype == "f32" else torch.bfloat16
    run = State(cfg, to_dev(synth.init_rows(W, 0, W.rows[0])).to(tdt),
                to_dev(synth.init_rows(W, 1, W.rows[1])).to(tdt))
    ws = N.Workspace(cfg)
    inputs = []
    for win in range(4):
        toks, dys = window_inputs(W, 4 * win)
        inputs.append(([to_dev(x) for x in toks], [to_dev(x) for x in dys]))
    saved = None
    for win in range(4):
        _window(N, cfg, run, ws, *inputs[win], win + 1)
        if win == 1:   # a checkpoint on the host: tables, row state, next step number
            torch.cuda.synchronize()
            saved = ([x.cpu() for x in run.W], [x.cpu() for x in run.st], win + 2)
    torch.cuda.synchronize()
    Ws, sts, t_next = saved
    res = State(cfg, Ws[0].cuda(), Ws[1].cuda())
    res.st = [x.cuda() for x in sts]
    ws2 = N.Workspace(cfg)
    for win in range(2, 4):
        _window(N, cfg, res, ws2, *inputs[win], t_next + win - 2)
    torch.cuda.synchronize()
    for c in range(2):
        assert torch.equal(run.W[c].view(torch.int16 if dtype == "bf16" else torch.int32),
                           res.W[c].view(torch.int16 if dtype == "bf16" else torch.int32)), c
        assert torch.equal(run.st[c].view(torch.int32), res.st[c].view(torch.int32)), c
    assert int((res.tl[0] == 4).sum()) > 0
    assert not np.array_equal(run.W[0].cpu().float().numpy(), Ws[0].float().numpy())
    assert N.device_status(cfg, ws) == 0 and N.device_status(cfg, ws2) == 0
