"""The sampled-softmax oracle's pins catch plausible mistakes: each case below
plants one mistake in the oracle (on the CPU, by replacing one of its
functions for the duration of the case) and checks that at least one pin of
tests/test_oracle_ssm.py then fails."""
import numpy as np
import pytest

import test_oracle_ssm as pins
from oracle import ssm

ORIG = {name: getattr(ssm, name) for name in ("candidates", "loss_fwd", "dlogits", "loss_bwd", "dW_rows")}


def _fill_ascending(targets, perm, V, C):
    # absent ids in ascending order instead of permutation order
    return ORIG["candidates"](targets, np.arange(V), V, C)


def _present_in_perm_order(targets, perm, V, C):
    cand, slot, n, ok = ORIG["candidates"](targets, perm, V, C)
    if not ok:
        return cand, slot, n, ok
    order = np.argsort(np.argsort(perm)[cand[:n]], kind="stable")   # present ids by permutation rank
    new = cand.copy()
    new[:n] = cand[:n][order]
    inv = np.empty(n, np.int64)
    inv[order] = np.arange(n)
    return new, inv[slot], n, ok


def _loss_over_vocab(X, W, cand, slot, chunk=4096):
    # normalises over the whole vocabulary instead of the candidate set
    V = len(W)
    full = np.arange(V)
    loss, lse = ORIG["loss_fwd"](X, W, full, np.asarray(cand)[np.asarray(slot)], chunk)
    return loss, lse


def _dlogits_no_g(X, W, cand, slot, dloss, lse=None):
    return ORIG["dlogits"](X, W, cand, slot, np.ones_like(np.asarray(dloss, np.float64)), lse)


def _dlogits_shifted_onehot(X, W, cand, slot, dloss, lse=None):
    return ORIG["dlogits"](X, W, cand, (np.asarray(slot) + 1) % len(cand), dloss, lse)


def _bwd_wrong_sign(X, W, cand, slot, dloss):
    dX, dWc = ORIG["loss_bwd"](X, W, cand, slot, dloss)
    return dX, -dWc


def _bwd_dx_from_unsorted_rows(X, W, cand, slot, dloss):
    dX, dWc = ORIG["loss_bwd"](X, W, cand, slot, dloss)
    dz = ssm.dlogits(X, W, cand, slot, dloss)
    return dz @ np.asarray(W, np.float64)[np.sort(cand)], dWc


MUTATIONS = [
    ("candidates", _fill_ascending, [pins.test_candidates_golden, pins.test_candidate_set_properties]),
    ("candidates", _present_in_perm_order, [pins.test_candidates_golden, pins.test_candidate_set_properties]),
    ("loss_fwd", _loss_over_vocab, [pins.test_sampled_loss_is_cross_entropy_over_the_candidates,
                                    pins.test_closed_forms]),
    ("dlogits", _dlogits_no_g, [pins.test_backward_is_torch_autograd, pins.test_dlogits_rows_sum_to_zero]),
    ("dlogits", _dlogits_shifted_onehot, [pins.test_backward_is_torch_autograd,
                                          pins.test_dlogits_rows_sum_to_zero]),
    ("loss_bwd", _bwd_wrong_sign, [pins.test_backward_is_torch_autograd,
                                   pins.test_backward_matches_central_differences]),
    ("loss_bwd", _bwd_dx_from_unsorted_rows, [pins.test_backward_is_torch_autograd]),
]


def _run_pin(pin):
    """Runs a pin with its parametrisations; True if all of them pass."""
    import inspect
    params = inspect.signature(pin).parameters
    cases = [{}]
    if "k" in params:
        cases = [{"k": k} for k in range(5)]
    elif "seed" in params:
        cases = [{"seed": s} for s in range(6)]
    try:
        for kw in cases:
            pin(**kw)
    except AssertionError:
        return False
    return True


@pytest.mark.parametrize("i", range(len(MUTATIONS)))
def test_a_planted_mistake_fails_a_pin(i, monkeypatch):
    name, bad, which = MUTATIONS[i]
    assert all(_run_pin(p) for p in which)          # the pins pass on the oracle as it is
    monkeypatch.setattr(ssm, name, bad)
    assert not all(_run_pin(p) for p in which), f"{bad.__name__} went unnoticed"
