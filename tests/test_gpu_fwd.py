"""GPU parity of context + hash and the signed gather-sum forward against the
oracle (bit-exact), through the C ABI.  Hashed bigram + trigram rows with a
sign trick: modded-nanogpt README, technique list."""
import numpy as np
import pytest
import torch

import helpers
import oracle
from gpu_common import device_table, host_rows, ng, to_dev
from sparse_hashed_gram_amd import synth, workloads

pytestmark = pytest.mark.gpu


def _idx_split(idx):
    u = idx.cpu().numpy().view(np.uint32)
    return (u[0] & 0x7FFFFFFF).astype(np.int64), (u[0] >> 31).astype(np.uint8), \
        (u[1] & 0x7FFFFFFF).astype(np.int64), (u[1] >> 31).astype(np.uint8)


@pytest.mark.parametrize("T", [1, 2, 3, 63, 64, 65, 255, 1000, 2048])
def test_hash_tiny_ragged(T):
    w = workloads.TINY
    N = ng()
    cfg = N.config(w.vocab, w.eos_id, w.rows, "f32", max_tokens=2048)
    tok = synth.tokens(w, 0)[:T]
    got = _idx_split(N.hash(cfg, to_dev(tok)))
    want = helpers.oracle_rows(w, tok, w.rows)
    for g, o in zip(got, want):
        np.testing.assert_array_equal(g, o)


@pytest.mark.parametrize("wl", [workloads.SHARD, workloads.FULL, workloads.COLLISION])
def test_hash_full_size_rows(wl):
    # hashing needs no table: check every position of a full micro-step
    N = ng()
    cfg = N.config(wl.vocab, wl.eos_id, wl.rows, wl.dtype, max_tokens=wl.tokens_per_step)
    tok = synth.tokens(wl, 1)
    got = _idx_split(N.hash(cfg, to_dev(tok)))
    want = helpers.oracle_rows(wl, tok, wl.rows)
    for g, o in zip(got, want):
        np.testing.assert_array_equal(g, o)


def test_hash_seeds_and_odd_row_counts():
    w = workloads.TINY
    N = ng()
    rows = (1, 3_000_017)
    cfg = N.config(w.vocab, w.eos_id, rows, "f32", seeds=(0xDEADBEEF12345678, 7), max_tokens=4096)
    tok = synth.tokens(w, 5)
    got = _idx_split(N.hash(cfg, to_dev(tok)))
    want = helpers.oracle_rows(w, tok, rows, seeds=(0xDEADBEEF12345678, 7))
    for g, o in zip(got, want):
        np.testing.assert_array_equal(g, o)
    assert (got[0] == 0).all()


def test_forward_tiny_f32_all_steps():
    w = workloads.TINY
    N = ng()
    cfg = N.config(w.vocab, w.eos_id, w.rows, "f32", max_tokens=w.tokens_per_step)
    Wb = synth.init_rows(w, 0, w.rows[0])
    Wt = synth.init_rows(w, 1, w.rows[1])
    Wb_d, Wt_d = to_dev(Wb), to_dev(Wt)
    for s in range(w.steps):
        tok = synth.tokens(w, s)
        out = N.embed_fwd(cfg, Wb_d, Wt_d, to_dev(tok)).cpu().numpy()
        rb, nb, rt, nt = helpers.oracle_rows(w, tok, w.rows)
        ref = oracle.forward(Wb, Wt, rb, nb, rt, nt, out_dtype="f32")
        np.testing.assert_array_equal(out.view(np.uint32), ref.view(np.uint32))


@pytest.mark.parametrize("T", [1, 65, 4097, 49_152])
def test_forward_shard_bf16(T):
    w = workloads.SHARD
    N = ng()
    cfg = N.config(w.vocab, w.eos_id, w.rows, "bf16", max_tokens=w.tokens_per_step)
    Wb = device_table(w.rows[0], "bf16", 11)
    Wt = device_table(w.rows[1], "bf16", 12)
    tok = synth.tokens(w, 3)[:T]
    out = N.embed_fwd(cfg, Wb, Wt, to_dev(tok))
    out = out.view(torch.int16).cpu().numpy().view(np.uint16)
    rb, nb, rt, nt = helpers.oracle_rows(w, tok, w.rows)
    ib, it = np.unique(rb), np.unique(rt)
    ref = oracle.forward(host_rows(Wb, ib), host_rows(Wt, it), rb, nb, rt, nt, ids_b=ib, ids_t=it,
                         out_dtype="bf16")
    np.testing.assert_array_equal(out, ref)
    del Wb, Wt
    torch.cuda.empty_cache()


@pytest.mark.parametrize("case", ["all_eos", "one_token", "two_tokens", "max_id"])
def test_forward_degenerate_streams(case):
    w = workloads.TINY
    N = ng()
    T = 3000
    cfg = N.config(w.vocab, w.eos_id, w.rows, "f32", max_tokens=T)
    tok = {"all_eos": np.full(T, w.eos_id, np.int32),
           "one_token": np.full(T, 17, np.int32),
           "two_tokens": np.tile(np.array([5, 9], np.int32), T // 2),
           "max_id": np.full(T, w.vocab - 1, np.int32)}[case]
    Wb = synth.init_rows(w, 0, w.rows[0])
    Wt = synth.init_rows(w, 1, w.rows[1])
    ws = N.Workspace(cfg)
    out = N.embed_fwd(cfg, to_dev(Wb), to_dev(Wt), to_dev(tok), ws=ws).cpu().numpy()
    rb, nb, rt, nt = helpers.oracle_rows(w, tok, w.rows)
    ref = oracle.forward(Wb, Wt, rb, nb, rt, nt)
    np.testing.assert_array_equal(out.view(np.uint32), ref.view(np.uint32))
    assert N.device_status(cfg, ws) == 0


def test_forward_bad_ids_flagged_and_consistent():
    w = workloads.TINY
    N = ng()
    T = 512
    cfg = N.config(w.vocab, w.eos_id, w.rows, "f32", max_tokens=T)
    tok = synth.tokens(w, 6)[:T].copy()
    tok[[10, 200]] = [-5, w.vocab + 3]
    Wb = synth.init_rows(w, 0, w.rows[0])
    Wt = synth.init_rows(w, 1, w.rows[1])
    ws = N.Workspace(cfg)
    out = N.embed_fwd(cfg, to_dev(Wb), to_dev(Wt), to_dev(tok), ws=ws).cpu().numpy()
    assert N.device_status(cfg, ws, clear=True) & N.FLAG_BAD_TOKEN
    assert N.device_status(cfg, ws) == 0
    rb, nb, rt, nt = helpers.oracle_rows(w, tok, w.rows)
    ref = oracle.forward(Wb, Wt, rb, nb, rt, nt)
    np.testing.assert_array_equal(out.view(np.uint32), ref.view(np.uint32))


def test_forward_empty_is_noop():
    w = workloads.TINY
    N = ng()
    cfg = N.config(w.vocab, w.eos_id, w.rows, "f32", max_tokens=16)
    Wb = torch.zeros((w.rows[0], 768), device="cuda")
    Wt = torch.zeros((w.rows[1], 768), device="cuda")
    out = N.embed_fwd(cfg, Wb, Wt, torch.zeros(0, dtype=torch.int32, device="cuda"))
    assert out.shape == (0, 768)


@pytest.mark.parametrize("T", [1, 65, 4097, 49_152])
def test_forward_shard_bf16_table_fp32_output(T):
    # NGRAM_OPT_OUT_F32: the exact fp32 sum of the two signed bf16 rows, not
    # rounded again; its bf16 rounding is the default output
    w = workloads.SHARD
    N = ng()
    cfg = N.config(w.vocab, w.eos_id, w.rows, "bf16", max_tokens=w.tokens_per_step, out_f32=True)
    cfg16 = N.config(w.vocab, w.eos_id, w.rows, "bf16", max_tokens=w.tokens_per_step)
    Wb = device_table(w.rows[0], "bf16", 13)
    Wt = device_table(w.rows[1], "bf16", 14)
    tok = synth.tokens(w, 4)[:T]
    out = N.embed_fwd(cfg, Wb, Wt, to_dev(tok))
    assert out.dtype == torch.float32
    out16 = N.embed_fwd(cfg16, Wb, Wt, to_dev(tok))
    assert torch.equal(out.to(torch.bfloat16), out16)
    rb, nb, rt, nt = helpers.oracle_rows(w, tok, w.rows)
    ib, it = np.unique(rb), np.unique(rt)
    ref = oracle.forward(host_rows(Wb, ib), host_rows(Wt, it), rb, nb, rt, nt, ids_b=ib, ids_t=it,
                         out_dtype="f32")
    np.testing.assert_array_equal(out.cpu().numpy().view(np.uint32), ref.view(np.uint32))
    del Wb, Wt
    torch.cuda.empty_cache()
