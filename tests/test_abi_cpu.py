"""CPU checks of the C ABI: the library loads, exports every entry point the
header declares, and rejects bad arguments on the host (before any HIP call,
so no GPU is needed)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ngram.h")


@pytest.fixture(scope="module")
def N():
    from sparse_hashed_gram_amd import ngram
    return ngram


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(ngram_[a-z_]+)\s*\(", src)))


def test_exports_every_declared_symbol(N):
    names = _declared()
    assert len(names) >= 12
    L = ctypes.CDLL(N._LIB_PATH)
    for n in names:
        assert hasattr(L, n), f"{n} declared in ngram.h but not exported"


def test_config_struct_layout(N):
    # the binding's ctypes mirror of ngram_config must match the C layout
    assert ctypes.sizeof(N.NgramConfig) == 80
    assert N.NgramConfig.dy_dtype.offset == 72


def test_version_and_status_strings(N):
    assert N.lib().ngram_abi_version() == 10
    for s in (0, -1, -2, -3, -4, -5, -6):
        assert N.status_string(s) not in ("", "unknown status")
    assert N.status_string(-99) == "unknown status"


def _good(N, **kw):
    args = dict(vocab=50304, eos_id=50256, rows=(4096, 4096), dtype="f32", max_tokens=2048)
    args.update(kw)
    return N.config(**args)


@pytest.mark.parametrize("field,value", [
    ("vocab", 0), ("eos_id", -1), ("eos_id", 50304), ("dim", 512), ("dtype", 2),
    ("max_tokens", 0), ("max_tokens", (1 << 28) + 1), ("accum_steps", 0), ("accum_steps", 65),
    ("mode", 3), ("window_rows", -1), ("dy_dtype", 2), ("dy_dtype", -1), ("options", 16), ("options", 1)])
def test_config_rejects(N, field, value):
    c = _good(N)
    setattr(c, field, value)
    assert N.config_check(c) == -3


def test_presort_is_for_burst_modes(N):
    assert N.config_check(_good(N, mode="burst_ref", presort=True)) == 0
    assert N.config_check(_good(N, mode="burst", presort=True)) == 0
    assert N.config_check(_good(N, mode="spread", presort=True)) == -3


def test_direct_table_needs_a_row_per_id(N):
    assert N.config_check(_good(N, rows=(50304, 1), direct=True)) == 0
    assert N.config_check(_good(N, rows=(50303, 1), direct=True)) == -3


def test_direct_table_takes_no_second_table(N):
    L = N.lib()
    c = _good(N, rows=(50304, 1), direct=True)
    fake = ctypes.c_void_p(1 << 40)
    # NULL W_t / state_t pass the host checks in direct mode (T out of range stops the call)
    assert L.ngram_embed_fwd(ctypes.byref(c), fake, None, fake, 5000, fake, None, None) == -4
    h = _good(N)
    assert L.ngram_embed_fwd(ctypes.byref(h), fake, None, fake, 5, fake, None, None) == -1


def test_config_rejects_rows(N):
    for r in (0, -1, 2**31):
        c = _good(N)
        c.rows[1] = r
        assert N.config_check(c) == -3
    c = _good(N, max_tokens=1 << 28, accum_steps=8, mode="burst")
    assert N.config_check(c) == -3       # burst positions must fit 30 bits
    assert N.config_check(_good(N, max_tokens=1 << 28, accum_steps=8)) == 0


def test_workspace_bytes_scale(N):
    small = N.workspace_bytes(_good(N))
    full = N.workspace_bytes(_good(N, rows=(42_300_000, 42_300_000), dtype="bf16", max_tokens=393_216))
    burst = N.workspace_bytes(_good(N, rows=(42_300_000, 42_300_000), dtype="bf16", max_tokens=393_216,
                                    mode="burst"))
    assert small < 64 << 20
    # window accumulator 2 x 1,572,864 x 3 KB dominates; slot maps 2 x 338 MB
    assert 10.2e9 < full < 11.0e9
    # burst keeps the window's dY (1,572,864 x 3 KB more; half that for bf16 dY)
    assert burst - full > 4.8e9
    burst16 = N.workspace_bytes(_good(N, rows=(42_300_000, 42_300_000), dtype="bf16", max_tokens=393_216,
                                      mode="burst", dy_dtype="bf16"))
    assert abs((burst - burst16) - 1_572_864 * 768 * 2) < 1 << 20


def test_host_rejections_enqueue_nothing(N):
    L = N.lib()
    c = _good(N)
    cp = ctypes.byref(c)
    fake = ctypes.c_void_p(1 << 40)           # never dereferenced: rejected first
    # T out of range
    assert L.ngram_hash(cp, fake, 4096, fake, None, None) == -4
    assert L.ngram_hash(cp, fake, -1, fake, None, None) == -4
    # null pointers
    assert L.ngram_hash(cp, None, 5, fake, None, None) == -1
    assert L.ngram_embed_fwd(cp, None, fake, fake, 5, fake, None, None) == -1
    assert L.ngram_embed_bwd_accum(cp, None, fake, fake, 5, None) == -1
    # misalignment
    assert L.ngram_embed_fwd(cp, ctypes.c_void_p((1 << 40) + 8), fake, fake, 5, fake, None, None) == -2
    assert L.ngram_workspace_init(cp, ctypes.c_void_p((1 << 40) + 128), 1 << 30, None) == -2
    # workspace too small
    assert L.ngram_workspace_init(cp, fake, 1024, None) == -4
    # step arguments
    ok = [fake] * 5
    assert L.ngram_sparse_step(cp, *ok, 0, 0.01, 0.95, 1e-8, None) == -5      # t < 1
    assert L.ngram_sparse_step(cp, *ok, 1, 0.01, 1.0, 1e-8, None) == -5       # beta2 = 1
    assert L.ngram_sparse_step(cp, *ok, 1, 0.01, -0.1, 1e-8, None) == -5
    assert L.ngram_sparse_step(cp, *ok, 1, 0.01, 0.95, 0.0, None) == -5       # eps = 0
    assert L.ngram_sparse_step(cp, *ok, 1, float("nan"), 0.95, 1e-8, None) == -5
    assert L.ngram_sparse_step(cp, *ok, 1, 0.01, 0.95, float("inf"), None) == -5
    # device step parameters: pointer required and 16-byte aligned
    assert L.ngram_sparse_step_dev(cp, *ok, None, None) == -1
    assert L.ngram_sparse_step_dev(cp, *ok, ctypes.c_void_p((1 << 40) + 4), None) == -2
    assert L.ngram_embed_bwd_step_dev(cp, fake, fake, fake, 5, *[fake] * 4, None, None) == -1
    # touched-rows arguments
    assert L.ngram_touched_rows(cp, fake, 2, fake, 10, fake, None) == -5
    assert L.ngram_touched_rows(cp, fake, 0, fake, -1, fake, None) == -4
    assert L.ngram_touched_rows(cp, fake, 0, None, 10, fake, None) == -1
    assert L.ngram_touched_rows(cp, fake, 0, fake, 10, None, None) == -1
    assert L.ngram_touched_rows(cp, fake, 0, fake, 10, ctypes.c_void_p((1 << 40) + 4), None) == -2
    # export arguments
    assert L.ngram_window_export(cp, fake, 2, fake, None, 10, fake, None) == -5
    assert L.ngram_window_export(cp, fake, 0, fake, None, -1, fake, None) == -4
    # bad config short-circuits everything
    c.dim = 7
    assert L.ngram_embed_fwd(cp, fake, fake, fake, 5, fake, None, None) == -3


@pytest.mark.parametrize("n_micro,T", [(1, 65_536), (64, 1_024), (63, 1_025), (3, 16_385), (4, 16_384)])
@pytest.mark.parametrize("dy_dtype", ["f32", "bf16"])
def test_noalloc_largest_windows_fit(N, n_micro, T, dy_dtype):
    # every window the allocation-free call accepts fits its fixed array:
    # the largest ones (65,536 positions, or the widest dY-row codes) on the
    # full-size tables with the nested sort pass every size check and reach
    # the first HIP call, which fails here, where no GPU is visible
    import torch
    if torch.cuda.device_count() > 0:
        pytest.skip("fake pointers: only where no GPU is visible")
    c = _good(N, rows=(42_300_000, 42_300_000), dtype="bf16", max_tokens=T, dy_dtype=dy_dtype, nest_always=True)
    fake = ctypes.c_void_p(1 << 40)
    rc = N.lib().ngram_window_step_noalloc(ctypes.byref(c), fake, fake, T, n_micro, fake, fake, fake, fake, 1,
                                           0.01, 0.95, 1e-8, None, None)
    assert rc == -6


def test_noalloc_window_host_rejections(N):
    # the allocation-free window step checks every size and pointer before
    # any HIP call (sizes beyond its fixed array are refused, not truncated)
    L = N.lib()
    c = _good(N)
    cp = ctypes.byref(c)
    fake = ctypes.c_void_p(1 << 40)
    tabs = [fake] * 4

    def call(T, n, *rest, tok=fake, dy=fake, t=1, beta2=0.95, flags=None):
        return L.ngram_window_step_noalloc(cp, tok, dy, T, n, *(rest or tabs), t, 0.01, beta2, 1e-8, flags,
                                           None)

    assert call(16_385, 4) == -4           # 65,540 positions: more than the array holds
    assert call(65_537, 1) == -4
    assert call(100, 0) == -4              # n_micro outside [1, 64]
    assert call(100, 65) == -4
    assert call(-1, 1) == -4
    assert call(100, 4, tok=None) == -1
    assert call(100, 4, dy=ctypes.c_void_p((1 << 40) + 8)) == -2
    assert call(100, 4, fake, None, fake, fake) == -1      # W_t required for two tables
    assert call(100, 4, flags=ctypes.c_void_p((1 << 40) + 2)) == -2
    assert call(100, 4, t=0) == -5
    assert call(100, 4, beta2=1.0) == -5
    assert call(0, 4) == 0                 # an empty window: nothing to do, nothing enqueued
