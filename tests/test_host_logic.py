"""CPU checks of the host-side logic around the path: the seeded synthetic
inputs (the stand-ins for the pages' FineWeb token streams) and the bench's
algorithmic-byte accounting, which turns measured kernel times into the
reported roofline fraction."""
import numpy as np
import pytest

import bench
from sparse_hashed_gram_amd import synth, workloads


# ------------------------------------------------------------ inputs

def test_zipf_cdf_is_the_normalised_power_law():
    cdf = synth.zipf_cdf(1000, 1.1)
    assert np.all(np.diff(cdf) > 0) and cdf[-1] == 1.0
    h = np.sum(np.arange(1, 1001, dtype=np.float64) ** -1.1)
    assert abs(cdf[0] - 1.0 / h) < 1e-15
    assert abs((cdf[9] - cdf[8]) - 10.0 ** -1.1 / h) < 1e-15


def test_tokens_are_seeded_and_in_range():
    w = workloads.FULL
    a = synth.tokens(w, 3, 50_000)
    b = synth.tokens(w, 3, 50_000)
    c = synth.tokens(w, 4, 50_000)
    assert a.dtype == np.int32 and np.array_equal(a, b) and not np.array_equal(a, c)
    assert a.min() >= 0 and a.max() < w.vocab


def test_zipf_ranks_follow_the_law():
    # id = rank - 1: the most frequent ids are the smallest, at Zipf(1.1) rates
    w = workloads.FULL
    t = synth.tokens(w, 0, 393_216)
    t = t[t != w.eos_id]
    h = np.sum(np.arange(1, w.vocab + 1, dtype=np.float64) ** -1.1)
    for r in (1, 2, 10):
        p = r ** -1.1 / h
        f = np.mean(t == r - 1)
        assert abs(f - p) < 6 * np.sqrt(p * (1 - p) / len(t)) + 1e-3


def test_documents_start_with_eos_and_respect_the_maximum_length():
    w = workloads.FULL
    t = synth.tokens(w, 1)
    assert t[0] == w.eos_id
    starts = np.flatnonzero(t == w.eos_id)
    gaps = np.diff(np.r_[starts, len(t)])
    assert gaps.max() <= w.doc_max
    # Geometric(1/1024) lengths clipped to [2, 2048]: mean length about 1,024 minus the clip
    assert 500 < len(t) / len(starts) < 1100


def test_fixed_layout_puts_eos_every_512():
    w = workloads.TINY
    t = synth.tokens(w, 0)
    assert np.all(t[::512] == w.eos_id)


def test_hot_set_and_collision_stream():
    w = workloads.COLLISION
    hs = synth.hot_set(w)
    assert len(hs) == 256 and len(np.unique(hs)) == 256 and w.eos_id not in hs
    assert np.array_equal(hs, synth.hot_set(w))
    t = synth.tokens(w, 0, 200_000)
    frac = np.mean(np.isin(t, hs))
    assert frac > 0.2 - 0.01   # 20 % replaced, plus the Zipf mass that falls on the hot ids


def test_dy_is_standard_normal_float32():
    w = workloads.SHARD
    d = synth.dY(w, 2, 4096)
    assert d.dtype == np.float32 and d.shape == (4096, 768)
    assert np.array_equal(d, synth.dY(w, 2, 4096))
    assert abs(float(d.mean())) < 0.01 and abs(float(d.std()) - 1.0) < 0.01


# ------------------------------------------------- algorithmic bytes

# A hand-made window of two micro-steps of T = 10 positions.  Per micro-step
# and channel: (distinct rows, rows new to the window, trigram rows that occur
# once and are new to the window, trigram rows that occur once).
STEPS = [[(6, 6, 0, 0), (9, 9, 8, 8)],
         [(5, 2, 0, 0), (10, 7, 5, 6)]]
UWIN = [8, 16]       # distinct rows of the window per channel
TSINGLE = 12         # trigram rows that occur once in the whole window
STATS = (STEPS, UWIN, TSINGLE)
T = 10
ROW = 1536           # bf16 table row
TS = 2 * ROW + 16    # table row read + written, state read + written


@pytest.mark.parametrize("dy_row", [3072, 1536])
def test_bytes_burst_by_reference(dy_row):
    b = bench.algorithmic_bytes(T, STATS, ROW, "burst_ref", "fused", dy_row, radix_passes=3)
    mn, kn = b["min"], b["kernel"]
    assert mn["fwd"] == kn["fwd"] == [T * (3 * ROW + 4)] * 2
    assert mn["stash"] == [T * 16] * 2              # token, two indices, row code
    assert mn["sort"] == [2 * 20 * 16 * 3]
    # the method's minimum: every dY row once, both channels' row ids, every
    # distinct row of either channel stepped once
    assert mn["reduce"] == [20 * dy_row + 24 * TS + 20 * 8]
    # the kernels: every bigram key and every trigram key but the window's
    # singletons read their dY row
    assert kn["reduce"] == [(40 - 12) * dy_row + 24 * TS + 20 * 8]
    assert mn["step"] == kn["step"] == [0]


def test_bytes_copying_burst_adds_the_dy_copy():
    b = bench.algorithmic_bytes(T, STATS, ROW, "burst", "fused", 3072, radix_passes=3)
    assert b["min"]["stash"] == b["kernel"]["stash"] == [T * (2 * 3072 + 16)] * 2


def test_bytes_spread_fused_last():
    b = bench.algorithmic_bytes(T, STATS, ROW, "spread", "fused", 3072, radix_passes=2)
    mn, kn = b["min"], b["kernel"]
    assert mn["sort"] == [2 * T * 16 * 2] * 2
    # micro-step 0 (accumulating): new rows written (3 KB), rows already there
    # read and written (6 KB); the method reads each dY row once, the kernels
    # read it for every key but the micro-step's trigram singletons
    win0 = 6 * 3072 + 0 + 9 * 3072 + 0
    m0_min = T * 3072 + win0 + T * 8
    m0_k = (T - 0) * 3072 + (T - 8) * 3072 + win0 + T * 8
    # micro-step 1 (fused with the step): rows already in the window read
    # their window row; every row it touches is stepped; the kernels read dY
    # for every key but the trigram rows that are singletons new to the window
    rows1 = 3 * 3072 + 5 * TS + 3 * 3072 + 10 * TS
    m1_min = T * 3072 + rows1 + T * 8
    m1_k = (T - 0) * 3072 + (T - 5) * 3072 + rows1 + T * 8
    assert mn["reduce"] == [m0_min, m1_min]
    assert kn["reduce"] == [m0_k, m1_k]
    # the separate step takes the window's other rows
    assert mn["step"] == kn["step"] == [(24 - 15) * (3072 + TS + 4)]


def test_bytes_spread_accumulate_then_step():
    b = bench.algorithmic_bytes(T, STATS, ROW, "spread", "accum", 3072, radix_passes=2)
    win1 = 2 * 3072 + 3 * 6144 + 7 * 3072 + 3 * 6144
    assert b["kernel"]["reduce"][1] == (T - 0) * 3072 + (T - 6) * 3072 + win1 + T * 8
    assert b["min"]["reduce"][1] == T * 3072 + win1 + T * 8
    assert len(b["min"]["reduce"]) == 2
    assert b["min"]["step"] == [24 * (3072 + TS + 4)]


def test_gpus_above_one_exit_with_a_message(capsys, monkeypatch):
    monkeypatch.setattr("sys.argv", ["bench.py", "--gpus", "2"])
    with pytest.raises(SystemExit) as e:
        bench.main()
    assert e.value.code == 2
    assert "one GPU" in capsys.readouterr().err


def test_kernel_code_hash_ignores_comments_only():
    # the PMC summaries are keyed by the kernel source's code: a comment or
    # layout edit keeps the key, any change to the code itself does not
    src = 'int f() { return 1; } // one\n/* block\n comment */ const char *s = "a // b";\n'
    assert bench.code_text(src) == 'int f() { return 1; } const char *s = "a // b";'
    assert bench.code_text(src.replace("// one", "// two")) == bench.code_text(src)
    assert bench.code_text(src.replace("return 1", "return 2")) != bench.code_text(src)
    assert bench.code_text("char c = '\\''; // x") == "char c = '\\'';"
    h = bench.src_hash("ngram_reduce.hip")
    assert len(h) == 16 and int(h, 16) >= 0
