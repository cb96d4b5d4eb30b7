"""GPU parity of nested trigram rows whose run of keys crosses the end of a
wavefront's walk in the fused reduction, against the oracle, through the C
ABI.

A trigram row whose positions all have one bigram row forms one contiguous
run in the bigram order, and the fused reduction's bigram pass sums it from
the dY rows it already loads (the trigram pass skips it).  A run inside a
bigram segment of many 64-key chunks is walked by several wavefronts: each
leaves its piece of the run, and the fix-up adds the pieces in order and
steps the row.  The windows here put one hot bigram (7, 8) after blocks of
repeated preceding tokens, so the runs have lengths 1 .. 2,500 and start and
end at every offset of the chunks (some exactly on chunk boundaries), cover
whole chunks, and exceed the 2,048-key tile of the trigram order (those rows
stay with the trigram pass).  Each micro-step uses its own preceding tokens,
so its trigram rows are new to the window (spread mode's fused last
micro-step nests only those).

Tolerances as in test_gpu_window: touched sets and t_last exact, v and W
within the bounds carried from the window-gradient bound; untouched rows
bitwise unchanged.
"""
import numpy as np
import pytest
import torch

from gpu_common import State, check_window, device_table, ng
from sparse_hashed_gram_amd import synth, workloads

pytestmark = pytest.mark.gpu

RUNS = [1, 2, 63, 64, 65, 127, 128, 129, 200, 1, 640, 64, 700, 2047, 2500, 3, 130]
ROWS = (1_000_003, 1_000_033)


def runs_tokens(m, hot=(7, 8)):
    """Micro-step m: EoS, then for each block i the tokens (a, 7, 8) repeated
    L_i times (a = 100 + 40 m + i, L_i the lengths rotated by m) with up to
    four random tokens between blocks."""
    rs = np.random.default_rng(900 + m)
    lengths = RUNS[m:] + RUNS[:m]
    out = [workloads.EOS_ID]
    for i, L in enumerate(lengths):
        out += [100 + 40 * m + i, hot[0], hot[1]] * L
        out += list(rs.integers(200, workloads.VOCAB, size=int(rs.integers(0, 5))))
    return np.asarray(out, np.int32)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("mode,how", [("burst_ref", "step"), ("burst", "step"), ("spread", "fused_last")])
def test_runs_across_walks(mode, how, dtype):
    w = workloads.TINY
    N = ng()
    toks = [runs_tokens(m) for m in range(4)]
    T = max(len(t) for t in toks)
    # windows this small take the nested sort only when asked to
    cfg = N.config(w.vocab, w.eos_id, ROWS, dtype, max_tokens=T, mode=mode, nest_always=True)
    st = State(cfg, device_table(ROWS[0], dtype, 71), device_table(ROWS[1], dtype, 72))
    ws = N.Workspace(cfg)
    for win in range(2):
        dys = [synth.dY(w, 700 + 4 * win + m, len(toks[m])) for m in range(4)]
        check_window(st, ws, toks, dys, win + 1, w.lr, w.beta2, w.eps, dtype, how=how)
        # the second window repeats the tokens: its rows are stepped again
    assert N.device_status(cfg, ws) == 0
    del st, ws
    torch.cuda.empty_cache()
