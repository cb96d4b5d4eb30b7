"""CPU oracle of the hashed bigram + trigram embedding path (ctypes front end).

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package.  The product path
(``sparse_hashed_gram_amd``) never imports it, and it never imports the
product path: the two share no code.  The arithmetic lives in
``ngram_oracle.c``; this module only marshals numpy arrays.

Every function cites the passage it follows in that C file's header.  The
sign-trick gather, the touched-rows-only update with beta1 = 0, one second
moment per 768-wide row, retroactive beta2 and 4-step accumulation come from
the modded-nanogpt README technique list and the @classiclarryd post quoted
on the airebao.com item about the 39.9 s record.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "ngram_oracle.c")
_LIB = os.path.join(_HERE, "libngram_oracle.so")

F32 = 0
BF16 = 1


def build(force: bool = False) -> str:
    """Compile the oracle with gcc (plain C11 + OpenMP)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-fopenmp", "-Wall", "-Wextra",
                               "-shared", "-fPIC", _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


class _Table(ctypes.Structure):
    _fields_ = [("dtype", ctypes.c_int32), ("pad", ctypes.c_int32),
                ("n_ids", ctypes.c_int64), ("ids", ctypes.c_void_p),
                ("data", ctypes.c_void_p)]


_lib = None


def lib():
    global _lib
    if _lib is None:
        # NGRAM_ORACLE_LIB: another build of this source (the mutation tests
        # load deliberately broken copies this way, in their own processes)
        L = ctypes.CDLL(os.environ.get("NGRAM_ORACLE_LIB") or build())
        u64, i64, i32, vp = ctypes.c_uint64, ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p
        L.orc_hash64.restype = u64
        L.orc_hash64.argtypes = [u64, u64]
        L.orc_row_of.restype = i64
        L.orc_row_of.argtypes = [u64, i64]
        L.orc_context.restype = None
        L.orc_context.argtypes = [vp, i64, i64, i32, vp, vp]
        L.orc_keys.restype = None
        L.orc_keys.argtypes = [i64, i64, i64, i32, vp, vp]
        L.orc_ngram_rows.restype = i64
        L.orc_ngram_rows.argtypes = [i64, i32, vp, vp, vp, i64, vp, vp, vp, vp]
        L.orc_double_to_bf16.restype = ctypes.c_uint16
        L.orc_double_to_bf16.argtypes = [ctypes.c_double]
        L.orc_bf16_to_double.restype = ctypes.c_double
        L.orc_bf16_to_double.argtypes = [ctypes.c_uint16]
        L.orc_forward.restype = ctypes.c_int
        L.orc_forward.argtypes = [ctypes.POINTER(_Table), ctypes.POINTER(_Table), i64,
                                  vp, vp, vp, vp, i64, vp, i32]
        L.orc_window_grad.restype = i64
        L.orc_window_grad.argtypes = [i64, i64, vp, vp, vp, vp, vp]
        L.orc_sparse_step.restype = None
        L.orc_sparse_step.argtypes = [i64, i64, vp, i32, vp, vp, vp, i32,
                                      ctypes.c_float, ctypes.c_float, ctypes.c_float]
        L.orc_threads.restype = ctypes.c_int
        L.orc_threads.argtypes = []
        L.orc_set_threads.restype = None
        L.orc_set_threads.argtypes = [ctypes.c_int]
        _lib = L
    return _lib


def _p(a: np.ndarray) -> int:
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data


def hash64(key: int, seed: int) -> int:
    return int(lib().orc_hash64(key, seed))


def row_of(z: int, R: int) -> int:
    return int(lib().orc_row_of(z, R))


def context(tok: np.ndarray, vocab: int, eos: int):
    tok = np.ascontiguousarray(tok, dtype=np.int32)
    p1 = np.empty(len(tok), np.int64)
    p2 = np.empty(len(tok), np.int64)
    lib().orc_context(_p(tok), len(tok), vocab, eos, _p(p1), _p(p2))
    return p1, p2


def keys(vocab: int, p2: int, p1: int, t: int):
    """(bigram key, trigram key) of one position."""
    kb = ctypes.c_uint64()
    kt = ctypes.c_uint64()
    lib().orc_keys(vocab, p2, p1, t, ctypes.addressof(kb), ctypes.addressof(kt))
    return int(kb.value), int(kt.value)


def ngram_rows(tok: np.ndarray, vocab: int, eos: int, rows, seeds=(1, 2)):
    """(row_b, neg_b, row_t, neg_t, n_bad) of one micro-step."""
    tok = np.ascontiguousarray(tok, dtype=np.int32)
    T = len(tok)
    R = np.asarray(rows, dtype=np.int64)
    S = np.asarray(seeds, dtype=np.uint64)
    rb = np.empty(T, np.int64)
    rt = np.empty(T, np.int64)
    nb = np.empty(T, np.uint8)
    nt = np.empty(T, np.uint8)
    bad = lib().orc_ngram_rows(vocab, eos, _p(R), _p(S), _p(tok), T,
                               _p(rb), _p(nb), _p(rt), _p(nt))
    return rb, nb, rt, nt, int(bad)


def double_to_bf16(x: float) -> int:
    return int(lib().orc_double_to_bf16(float(x)))


def bf16_to_double(h: int) -> float:
    return float(lib().orc_bf16_to_double(int(h)))


def _table(W: np.ndarray, ids: np.ndarray | None):
    dt = F32 if W.dtype == np.float32 else BF16
    if dt == BF16:
        assert W.dtype == np.uint16
    t = _Table(dt, 0, 0 if ids is None else len(ids),
               None if ids is None else _p(ids), _p(W))
    return t


def forward(Wb: np.ndarray, Wt: np.ndarray, rb, nb, rt, nt,
            ids_b: np.ndarray | None = None, ids_t: np.ndarray | None = None,
            out_dtype: str = "f32") -> np.ndarray:
    """Signed two-row gather-sum.  Tables are float32 or uint16 (bf16 bits),
    dense (ids None) or snapshots of the ascending rows ``ids``."""
    Wb = np.ascontiguousarray(Wb)
    Wt = np.ascontiguousarray(Wt)
    dim = Wb.shape[1]
    T = len(rb)
    rb, rt = (np.ascontiguousarray(a, np.int64) for a in (rb, rt))
    nb, nt = (np.ascontiguousarray(a, np.uint8) for a in (nb, nt))
    if ids_b is not None:
        ids_b = np.ascontiguousarray(ids_b, np.int64)
    if ids_t is not None:
        ids_t = np.ascontiguousarray(ids_t, np.int64)
    tb, tt = _table(Wb, ids_b), _table(Wt, ids_t)
    odt = F32 if out_dtype == "f32" else BF16
    out = np.empty((T, dim), np.float32 if odt == F32 else np.uint16)
    rc = lib().orc_forward(ctypes.byref(tb), ctypes.byref(tt), dim, _p(rb), _p(nb),
                           _p(rt), _p(nt), T, _p(out), odt)
    if rc != 0:
        raise KeyError("forward: a row is missing from a table snapshot")
    return out


def window_grad(rows: np.ndarray, neg: np.ndarray, dY: np.ndarray):
    """One channel's window gradient.  ``rows``/``neg``/``dY`` are the
    window's micro-steps concatenated in order.  Returns (touched ascending
    int64 [U], G float32 [U, dim])."""
    rows = np.ascontiguousarray(rows, np.int64)
    neg = np.ascontiguousarray(neg, np.uint8)
    dY = np.ascontiguousarray(dY, np.float32)
    N, dim = dY.shape
    assert len(rows) == N and len(neg) == N
    touched = np.empty(max(N, 1), np.int64)
    G = np.empty((max(N, 1), dim), np.float32)
    U = lib().orc_window_grad(dim, N, _p(rows), _p(neg), _p(dY), _p(touched), _p(G))
    return touched[:U].copy(), G[:U].copy()


def sparse_step(G: np.ndarray, W: np.ndarray, v: np.ndarray, t_last: np.ndarray,
                t: int, lr: float, beta2: float, eps: float):
    """Lazy row-wise Adam(beta1 = 0) step on touched rows; returns new copies
    of (W, v, t_last).  W is float32 or uint16 (bf16 bits), one row per
    touched row, aligned with G."""
    G = np.ascontiguousarray(G, np.float32)
    W = np.array(W, copy=True, order="C")
    v = np.array(v, dtype=np.float32, copy=True)
    tl = np.array(t_last, dtype=np.int32, copy=True)
    U, dim = G.shape
    wdt = F32 if W.dtype == np.float32 else BF16
    lib().orc_sparse_step(dim, U, _p(G), wdt, _p(W), _p(v), _p(tl), int(t),
                          float(lr), float(beta2), float(eps))
    return W, v, tl


def threads() -> int:
    return int(lib().orc_threads())


def set_threads(n: int) -> None:
    """Threads of the oracle's OpenMP loops (n <= 0: all processors)."""
    lib().orc_set_threads(int(n))
