"""Pins of the oracle's forward (signed two-row gather-sum) and its bf16
rounding (CPU only).

The forward is a plain sparse-dense product: with S_c the +/-1 selection
matrix of channel c, out = S_b W_b + S_t W_t (hashed bigram + trigram table
with sign trick, modded-nanogpt README technique list).  numpy's dense matmul
is an independent route to the same numbers.  Rounding to bf16 is pinned to
torch's CPU float->bfloat16 conversion (round to nearest even) and, for values
that are not floats, to a brute-force nearest search over all bf16 values.
"""
import numpy as np
import pytest
import torch

import oracle
from oracle import dense
from sparse_hashed_gram_amd import synth, workloads


def _bits_to_f32(u16: np.ndarray) -> np.ndarray:
    return (u16.astype(np.uint32) << 16).view(np.float32)


def _torch_bf16_bits(x_f32: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(x_f32, np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


# every positive finite bf16 value, ascending, plus +inf as the last candidate
_POS = np.arange(0x0000, 0x7F80, dtype=np.uint16)
_POS_VAL = _bits_to_f32(_POS).astype(np.float64)


def _brute_bf16(x: float) -> int:
    if x == 0:
        return 0x8000 if np.signbit(x) else 0
    s = 0x8000 if x < 0 else 0
    a = abs(x)
    vals = np.append(_POS_VAL, 2.0 ** 128)
    pats = np.append(_POS, np.uint16(0x7F80))
    j = np.searchsorted(vals, a)
    cands = [k for k in (j - 1, j) if 0 <= k < len(vals)]
    best = min(cands, key=lambda k: (abs(vals[k] - a), int(pats[k]) & 1))
    return s | int(pats[best])


def test_bf16_rne_matches_torch_on_floats():
    rs = np.random.default_rng(0)
    xs = np.concatenate([
        rs.standard_normal(20000).astype(np.float32) * np.float32(0.02),
        rs.standard_normal(5000).astype(np.float32) * np.float32(1e30),
        (rs.random(5000) * 2.0 ** -126).astype(np.float32),          # subnormal range
        np.array([0.0, -0.0, 1.0, -1.0, 3.0e38, -3.0e38, 1e-45, np.inf, -np.inf],
                 np.float32),
    ])
    # exact ties: bf16 value + half an ulp, both parities
    base = _bits_to_f32(rs.integers(0x0080, 0x7F00, size=4000).astype(np.uint16))
    ties = (base.view(np.uint32) | np.uint32(0x8000)).view(np.float32)
    xs = np.concatenate([xs, ties, -ties])
    want = _torch_bf16_bits(xs)
    got = np.array([oracle.double_to_bf16(float(x)) for x in xs], np.uint16)
    np.testing.assert_array_equal(got, want)


def test_bf16_rne_nan_and_overflow():
    assert oracle.double_to_bf16(float("nan")) == 0x7FC0
    max_bf16 = float(_bits_to_f32(np.array([0x7F7F], np.uint16))[0])
    half_ulp = 2.0 ** (127 - 8)
    assert oracle.double_to_bf16(max_bf16) == 0x7F7F
    assert oracle.double_to_bf16(max_bf16 + half_ulp * 0.99) == 0x7F7F
    assert oracle.double_to_bf16(max_bf16 + half_ulp) == 0x7F80   # tie -> even (inf)
    assert oracle.double_to_bf16(-(max_bf16 + 2 * half_ulp)) == 0xFF80


def test_bf16_rne_brute_force_on_doubles():
    # doubles between bf16 values (not representable as float), near ties
    rs = np.random.default_rng(1)
    pats = rs.integers(0x0001, 0x7F7F, size=300).astype(np.uint16)
    lo = _bits_to_f32(pats).astype(np.float64)
    hi = _bits_to_f32(pats + 1).astype(np.float64)
    mid = (lo + hi) / 2
    xs = np.concatenate([mid, mid * (1 + 2.0 ** -40), mid * (1 - 2.0 ** -40),
                         lo + (hi - lo) * rs.random(300)])
    xs = np.concatenate([xs, -xs, [2.0 ** -134, 2.0 ** -133 * 1.5, 2.0 ** -133 * 2.5]])
    for x in xs:
        assert oracle.double_to_bf16(float(x)) == _brute_bf16(float(x)), x
        assert oracle.bf16_to_double(oracle.double_to_bf16(float(x))) == \
            float(_bits_to_f32(np.array([_brute_bf16(float(x))], np.uint16))[0])


def _tiny_tables(R=(257, 311), dim=768, seed=3):
    rs = np.random.default_rng(seed)
    Wb = (rs.standard_normal((R[0], dim)) * 0.02).astype(np.float32)
    Wt = (rs.standard_normal((R[1], dim)) * 0.02).astype(np.float32)
    return Wb, Wt


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_forward_equals_dense_selection_product(dtype):
    w = workloads.TINY
    tok = synth.tokens(w, 0)[:700]
    R = (257, 311)
    Wb, Wt = _tiny_tables(R)
    if dtype == "bf16":
        Wb = _bits_to_f32(_torch_bf16_bits(Wb))
        Wt = _bits_to_f32(_torch_bf16_bits(Wt))
    rb, nb, rt, nt, _ = oracle.ngram_rows(tok, w.vocab, w.eos_id, R)
    ref = dense.forward(dense.selection_matrix(rb, nb, R[0]), Wb,
                        dense.selection_matrix(rt, nt, R[1]), Wt)
    ref32 = ref.astype(np.float32)   # exact sum of two table values, rounded once
    if dtype == "f32":
        got = oracle.forward(Wb, Wt, rb, nb, rt, nt, out_dtype="f32")
        np.testing.assert_array_equal(got.view(np.uint32), ref32.view(np.uint32))
    else:
        got = oracle.forward(_torch_bf16_bits(Wb), _torch_bf16_bits(Wt), rb, nb, rt, nt,
                             out_dtype="bf16")
        np.testing.assert_array_equal(got, _torch_bf16_bits(ref32))


def test_forward_snapshot_view_equals_dense_view():
    w = workloads.TINY
    tok = synth.tokens(w, 1)[:500]
    R = (300, 400)
    Wb, Wt = _tiny_tables(R, seed=4)
    rb, nb, rt, nt, _ = oracle.ngram_rows(tok, w.vocab, w.eos_id, R)
    full = oracle.forward(Wb, Wt, rb, nb, rt, nt)
    ib, it = np.unique(rb), np.unique(rt)
    snap = oracle.forward(Wb[ib], Wt[it], rb, nb, rt, nt, ids_b=ib, ids_t=it)
    np.testing.assert_array_equal(full, snap)
    with pytest.raises(KeyError):
        oracle.forward(Wb[ib[1:]], Wt[it], rb, nb, rt, nt, ids_b=ib[1:], ids_t=it)


def test_forward_sign_trick_cancels():
    # R = 1 sends every n-gram to row 0; a position whose two signs differ
    # reads W_b[0] - W_t[0]; equal signs read +/-(W_b[0] + W_t[0]).
    w = workloads.TINY
    tok = synth.tokens(w, 2)[:200]
    rb, nb, rt, nt, _ = oracle.ngram_rows(tok, w.vocab, w.eos_id, (1, 1))
    assert (rb == 0).all() and (rt == 0).all()
    Wb = np.full((1, 768), 0.25, np.float32)
    Wt = np.full((1, 768), 0.25, np.float32)
    out = oracle.forward(Wb, Wt, rb, nb, rt, nt)
    expect = np.where(nb != nt, 0.0, np.where(nb == 1, -0.5, 0.5)).astype(np.float32)
    np.testing.assert_array_equal(out[:, 0], expect)
    assert 0 < (nb != nt).mean() < 1
