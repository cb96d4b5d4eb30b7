"""Bounds of the fused reduction's indexing, checked on the CPU.

tests/kernel_model/seg_step_index.cpp walks the sorted keys of a burst
window exactly as seg_step_kernel's wavefronts do (the chunk plan, the
readlanes of keys 0..127, the dY row of each key from its micro-step and
position, the singleton map, table rows and state, window slots, partial
rows and fix-up records, the pieces and records of nested trigram runs that
cross a walk's end; then group_sum_kernel and fixup_kernel) and checks
every index against the extent of its buffer in the workspace layout.  It
also checks the bookkeeping the indexing serves: each key walked once, each
segment completed once, each trigram row the bigram pass completes stepped
once with each of its keys in exactly one completed sum, and every partial
row, group sum or run piece the fix-up reads written.

The windows are those of the GPU tests: the full Zipf 1.1 window and the
collision-stress window (4 x 393,216 positions, 42.3M rows per table), the
ragged window (262,143 / 100,000 / 7 / 150,001 positions), one hot row over
20,000 positions, and the token-indexed value-embedding window (hot ids of
more than 64 chunks' worth of keys: the fix-up's block-wide scan).  The
sorted keys, their payloads and the singleton map are built here the way the
library defines them (stable sort by row; payload = micro-step << pos_bits |
position with the sign in bit 31; a trigram row that occurs once in the
window is a singleton), from the oracle's rows.
"""
import ctypes
import os
import subprocess

import numpy as np
import pytest

import oracle
from sparse_hashed_gram_amd import synth, workloads

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "kernel_model", "seg_step_index.cpp")
NEW_HEAD = 0xFFFFFFFE
NOT_SINGLE = 0xFFFFFFFF


@pytest.fixture(scope="module")
def model(tmp_path_factory):
    lib = str(tmp_path_factory.mktemp("model") / "libsegmodel.so")
    subprocess.check_call(["g++", "-O2", "-std=c++17", "-shared", "-fPIC", SRC, "-o", lib])
    L = ctypes.CDLL(lib)
    vp, i64 = ctypes.c_void_p, ctypes.c_int64
    L.model_channel.restype = i64
    L.model_channel.argtypes = [i64, vp, vp, vp, i64, vp, i64, vp, ctypes.c_int, ctypes.c_int, vp, i64, i64, i64,
                                i64, i64, ctypes.c_int, ctypes.c_int, vp, vp, vp, vp, vp, vp, vp]
    return L


def _p(a):
    return None if a is None else a.ctypes.data


def _sorted_keys(rows, neg, codes):
    order = np.argsort(rows, kind="stable")
    R = rows[order].astype(np.uint32)
    V = (codes[order].astype(np.uint64) | (neg[order].astype(np.uint64) << 31)).astype(np.uint32)
    return R, V


def _run(model, n, R, V, I, nk, tinfo, code_cap, pos_bits, Tm, rows_c, rows_t, step_u=2, nested=False, tix=None):
    nchunk = (nk + 63) // 64
    ngroup = (nchunk + 63) // 64
    walked = np.zeros(max(n, 1), np.int32)
    completed = np.zeros(max(n, 1), np.int32)
    tstepped = np.zeros(code_cap, np.int32)
    tsum = np.zeros(code_cap, np.int32)
    acc = ctypes.c_int64()
    ntrec = ctypes.c_int64()
    msg = ctypes.create_string_buffer(256)
    Tm = np.ascontiguousarray(Tm, np.int64)
    wrows = min(max(rows_c, rows_t), nk)
    ext = np.zeros(nk, np.uint32)   # the arrays at their workspace extent (nk entries)
    Rx, Vx, Ix = ext.copy(), ext.copy(), ext.copy()
    Rx[:n], Vx[:n], Ix[:n] = R, V, I
    Xx = None
    if tix is not None:
        Xx = ext.copy()
        Xx[:n] = tix
    viol = model.model_channel(n, _p(Rx), _p(Vx), _p(Ix), nk, _p(tinfo), code_cap, _p(Xx), pos_bits, len(Tm), _p(Tm),
                               rows_c, rows_t, wrows, nchunk, ngroup, step_u, int(nested), _p(walked), _p(completed),
                               _p(tstepped), _p(tsum), ctypes.byref(ntrec), ctypes.byref(acc), msg)
    assert viol == 0, msg.value.decode()
    assert acc.value > 0 or n == 0
    _run.n_trec = ntrec.value
    return walked[:n], completed[:n], tstepped, tsum


def _heads(R):
    h = np.ones(len(R), bool)
    h[1:] = R[1:] != R[:-1]
    return h


MULTI, RUN_HEAD, RUN_TAIL = 0x40000000, 0x20000000, 0x10000000
TILE = 2048   # mark_kernel's tile of the trigram order


def _nested_records(Rt, Vt, rb_of_code, code_cap):
    """mark_kernel's decision on an empty window: a trigram row is completed
    by the bigram pass if its keys lie in one 2,048-key tile of the trigram
    order and all have the same bigram row.  Records: row | sign, and for a
    row of several keys MULTI with RUN_HEAD / RUN_TAIL on its first / last
    key; the map is indexed by the key's place in the trigram order.
    Returns (records, kept mask, nested mask, segment ids)."""
    n = len(Rt)
    idx = np.arange(n)
    head = _heads(Rt)
    end = np.ones(n, bool)
    end[:-1] = Rt[1:] != Rt[:-1]
    hidx = np.maximum.accumulate(np.where(head, idx, 0))
    eidx = np.minimum.accumulate(np.where(end, idx, n)[::-1])[::-1]
    seg = np.cumsum(head) - 1
    code = (Vt & 0x7FFFFFFF).astype(np.int64)
    bkey = rb_of_code[code].astype(np.int64)
    mism = np.zeros(n, bool)
    mism[1:] = (~head[1:]) & (bkey[1:] != bkey[:-1])
    fail = np.zeros(int(seg[-1]) + 1 if n else 0, bool)
    np.logical_or.at(fail, seg, mism)
    nested = ((hidx // TILE) == (eidx // TILE)) & ~fail[seg]
    single = head & end
    bits = np.where(single, 0, MULTI | np.where(head, RUN_HEAD, 0) | np.where(end, RUN_TAIL, 0))
    rec = np.where(nested, Rt | (Vt & 0x80000000) | bits, NOT_SINGLE).astype(np.uint32)
    tinfo = np.full(code_cap, NOT_SINGLE, np.uint32)
    tinfo[:n] = rec
    return tinfo, ~nested, nested, seg


def _check_window(model, toks, rows, max_tokens, direct=False):
    """Both channels of one burst-by-reference window, fused with the step:
    the bigram keys in (bigram row, trigram row, position) order, the
    trigram keys in (trigram row, position) order, nested trigram rows
    completed by the bigram pass."""
    A = len(toks)
    pos_bits = max(0, int(max_tokens - 1).bit_length())
    code_cap = A << pos_bits
    nk = A * max_tokens
    codes, rb, nb, rt, nt = [], [], [], [], []
    for m, tok in enumerate(toks):
        codes.append((np.uint64(m) << np.uint64(pos_bits)) | np.arange(len(tok), dtype=np.uint64))
        if direct:
            rb.append(tok.astype(np.int64))
            nb.append(np.zeros(len(tok), np.uint8))
        else:
            b, x, t, y, _ = oracle.ngram_rows(tok, workloads.VOCAB, workloads.EOS_ID, rows)
            rb.append(b); nb.append(x); rt.append(t); nt.append(y)
    codes = np.concatenate(codes)
    n = len(codes)
    Tm = [len(t) for t in toks]
    rb, nb = np.concatenate(rb), np.concatenate(nb)
    if direct:
        Rb, Vb = _sorted_keys(rb, nb, codes)
        Ib = np.where(_heads(Rb), NEW_HEAD, 0).astype(np.uint32)
        walked, completed, _, _ = _run(model, n, Rb, Vb, Ib, nk, None, code_cap, pos_bits, Tm, rows[0], 1)
        assert (walked == 1).all()
        np.testing.assert_array_equal(completed, _heads(Rb).astype(np.int32))
        return
    rt, nt = np.concatenate(rt), np.concatenate(nt)
    ot = np.argsort(rt, kind="stable")                    # trigram order
    obt = ot[np.argsort(rb[ot], kind="stable")]           # (bigram row, trigram row, position)
    Rb = rb[obt].astype(np.uint32)
    Vb = (codes[obt] | (nb[obt].astype(np.uint64) << 31)).astype(np.uint32)
    Ib = np.where(_heads(Rb), NEW_HEAD, 0).astype(np.uint32)
    Rt = rt[ot].astype(np.uint32)
    Vt = (codes[ot] | (nt[ot].astype(np.uint64) << 31)).astype(np.uint32)
    rb_of_code = np.zeros(code_cap, np.int64)
    rb_of_code[codes.astype(np.int64)] = rb
    tinfo, kept, nested, tseg = _nested_records(Rt, Vt, rb_of_code, code_cap)
    inv_ot = np.empty(n, np.int64)
    inv_ot[ot] = np.arange(n)
    tix = inv_ot[obt].astype(np.uint32)   # each bigram key's place in the trigram order
    walked, completed, tstepped, tsum = _run(model, n, Rb, Vb, Ib, nk, tinfo, code_cap, pos_bits, Tm, rows[0],
                                             rows[1], nested=True, tix=tix)
    _check_window.n_trec = _run.n_trec
    assert (walked == 1).all(), np.flatnonzero(walked != 1)[:10]
    np.testing.assert_array_equal(completed, _heads(Rb).astype(np.int32))
    # every nested trigram row is stepped exactly once by the bigram pass
    # (at one of its keys), no other row is
    per_row = np.bincount(tseg, weights=tstepped[(Vt & 0x7FFFFFFF).astype(np.int64)])
    nested_seg = np.zeros(len(per_row), bool)
    nested_seg[tseg[nested]] = True
    np.testing.assert_array_equal(per_row, nested_seg.astype(float))
    # each key of a nested row is in exactly one completed sum, no kept key is
    np.testing.assert_array_equal(tsum[(Vt & 0x7FFFFFFF).astype(np.int64)], nested.astype(np.int32))
    # the trigram pass walks the kept keys, in order, with their head info
    h = _heads(Rt)
    Rs, Vs = Rt[kept], Vt[kept]
    Is = np.where(h[kept], NEW_HEAD, 0).astype(np.uint32)
    w2, c2, _, _ = _run(model, len(Rs), Rs, Vs, Is, nk, None, code_cap, pos_bits, Tm, rows[1], rows[1])
    assert (w2 == 1).all()
    np.testing.assert_array_equal(c2, _heads(Rs).astype(np.int32))
    # every trigram row completed exactly once over both passes
    assert int(c2.sum()) + int(nested_seg.sum()) == int(h.sum())
    return int(kept.sum())


def test_full_window(model):
    w = workloads.FULL
    kept = _check_window(model, [synth.tokens(w, m) for m in range(4)], w.rows, w.tokens_per_step)
    assert kept < 80_000   # of 1,572,864 trigram keys, about 73K are left to the trigram pass
    assert _check_window.n_trec > 2000   # runs completed by the fix-up


def test_collision_window(model):
    w = workloads.COLLISION
    _check_window(model, [synth.tokens(w, m) for m in range(4)], w.rows, w.tokens_per_step)


def test_ragged_window(model):
    w = workloads.FULL
    Ts = [262_143, 100_000, 7, 150_001]
    _check_window(model, [synth.tokens(w, 20 + m, Ts[m]) for m in range(4)], w.rows, max(Ts))


@pytest.mark.parametrize("T", [65, 129, 4097, 20_000])
def test_single_hot_row(model, T):
    # one token repeated: every position hits the same bigram and trigram rows
    # (after the first two), segments of thousands of keys over many chunks
    toks = [np.full(T, 17, np.int32)]
    _check_window(model, toks, (4096, 4096), T)


def test_value_embedding_window(model):
    w = workloads.VALUE
    _check_window(model, [synth.tokens(w, m) for m in range(4)], (w.rows[0], 1), w.tokens_per_step, direct=True)


def test_the_model_reports_an_index_past_its_buffer(model):
    # the model itself: told that micro-step 0 has one position fewer than its
    # keys name, it must report that key's dY row as out of bounds
    tok = synth.tokens(workloads.TINY, 0, 300)
    rb, nb, _, _, _ = oracle.ngram_rows(tok, workloads.VOCAB, workloads.EOS_ID, (4096, 4096))
    codes = np.arange(300, dtype=np.uint64)
    R, V = _sorted_keys(rb, nb, codes)
    I = np.where(_heads(R), NEW_HEAD, 0).astype(np.uint32)
    with pytest.raises(AssertionError, match="dY position"):
        _run(model, 300, R, V, I, 300, None, 512, 9, [299], 4096, 4096)


def test_the_model_reports_a_split_run(model):
    # the model itself: a nested run whose keys are not adjacent in the walk
    # (a single key of the same row in between) must be reported
    R = np.array([5, 5, 5, 5], np.uint32)
    V = np.arange(4, dtype=np.uint32)
    I = np.array([NEW_HEAD, 0, 0, 0], np.uint32)
    tinfo = np.full(8, NOT_SINGLE, np.uint32)
    tinfo[0] = 9 | MULTI | RUN_HEAD
    tinfo[2] = 9 | MULTI | RUN_TAIL
    tinfo[1] = 9
    with pytest.raises(AssertionError, match="nested run"):
        _run(model, 4, R, V, I, 4, tinfo, 8, 3, [4], 16, 16, nested=True)


def test_the_model_reports_a_run_without_its_tail(model):
    # the model itself: a run over two chunks whose last key lacks RUN_TAIL
    # leaves a first piece that the fix-up cannot close
    n = 100
    R = np.full(n, 5, np.uint32)
    V = np.arange(n, dtype=np.uint32)
    I = np.zeros(n, np.uint32)
    I[0] = NEW_HEAD
    tinfo = np.full(128, NOT_SINGLE, np.uint32)
    tinfo[:n] = 9 | MULTI
    tinfo[0] |= RUN_HEAD
    with pytest.raises(AssertionError, match="run"):
        _run(model, n, R, V, I, n, tinfo, 128, 7, [n], 16, 16, nested=True)


def _runs_window(run_lengths, hot=(7, 8), seed=5):
    """Tokens where one bigram (hot) is preceded by one token per block of
    run_lengths[i] repetitions: trigram rows of run_lengths[i] keys each,
    all in the hot bigram's segment, so runs start and end at every offset
    of the 64-key chunks (some exactly at chunk boundaries), cover whole
    chunks, and cross the 2,048-key tile of the trigram order when longer."""
    rs = np.random.default_rng(seed)
    out = [0]
    for i, L in enumerate(run_lengths):
        a = 100 + i
        out += [a, hot[0], hot[1]] * L
        out += list(rs.integers(200, 50_000, size=int(rs.integers(0, 5))))
    return np.asarray(out, np.int32)


RUNS = [1, 2, 63, 64, 65, 127, 128, 129, 200, 1, 640, 64, 700, 2047, 2500, 3, 130]


@pytest.mark.parametrize("step_u", [2])
def test_runs_across_chunks(model, step_u):
    tok = _runs_window(RUNS)
    kept = _check_window(model, [tok, tok[: len(tok) // 2], tok[:7], tok], (4096, 4096), len(tok))
    # runs that cross a walk's end, completed by the fix-up, and runs too
    # long for one tile of the trigram order, left to the trigram pass
    assert _check_window.n_trec > 10
    assert kept > 2500
