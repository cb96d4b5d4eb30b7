#!/usr/bin/env python3
"""Benchmark of the hashed bigram + trigram embedding path on one MI355X.

One step = one accumulation window of the whole hot path: 4 micro-steps of
the forward (context + hash + signed gather-sum) and the backward (keys
kept), then the window's reduction fused with the lazy sparse step (sort,
dedupe, signed segment reduction, step of every touched row).  --mode
spread reduces each micro-step into the window accumulator as it comes and
fuses the step into the last one instead.  Workload (default): the full
84.6M-row table (2 x 42,300,000 x 768 bf16, about 130 GB) resident on one
GPU, 393,216 tokens per micro-step drawn from Zipf(1.1) over a 50,304-id
vocabulary with EoS-aligned documents (synthetic stand-in for FineWeb),
upstream gradients N(0, 1).

Prints one JSON line.  `value` is the window's tokens per second through the
whole path with all inputs resident in HBM; per-kernel-group times come from
HIP events recorded on the launch stream around each group inside the timed
region; `roofline` reports the dominant group's algorithmic bytes per launch
(the bytes the method cannot avoid moving: each upstream gradient row read
once, each touched row's table row and state read and written once, the row
ids) over its mean launch time against the 8 TB/s HBM3E peak; `cpu_baseline`
times the CPU oracle on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "updated rows/s + fwd tokens/s; achieved HBM GB/s vs peak, 84.6M-row table"
HBM_PEAK_GBPS = 8000.0
ROW_BF16 = 768 * 2
ROW_F32 = 768 * 4
GROUPS = ("fwd", "sort", "reduce", "step", "stash")
KERNEL_SRC = {"fwd": "ngram_fwd.hip", "sort": "ngram_reduce.hip", "reduce": "ngram_reduce.hip",
              "step": "ngram_step.hip", "stash": "ngram_fwd.hip",
              "ssm_fwd": "ssm.hip", "ssm_dz": "ssm.hip", "ssm_dx": "ssm.hip", "ssm_dw": "ssm.hip"}


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20, help="timed windows")
    ap.add_argument("--warmup", type=int, default=5, help="untimed windows")
    ap.add_argument("--workload", default="full", choices=["tiny", "shard", "full", "collision", "value", "ssm"],
                    help="ssm: the sampled-softmax loss (include/ssm.h) instead of the n-gram table; "
                         "one step = candidate set + loss forward + backward of one micro-batch")
    ap.add_argument("--candidates", type=int, default=10240,
                    help="ssm: candidate-set size (10240, 14336, 24576 or 50304 in the speedrun)")
    ap.add_argument("--ssm-tokens", type=int, default=49152,
                    help="ssm: positions per micro-batch (one GPU's share of the 393,216-token batch)")
    ap.add_argument("--mode", default="burst_ref", choices=["spread", "burst", "burst_ref"],
                    help="spread: each micro-step reduced into the window at once; burst: micro-steps "
                         "kept (dY copied) and reduced with the step; burst_ref: as burst, dY read "
                         "in place at step time")
    ap.add_argument("--dy-dtype", default="f32", choices=["f32", "bf16"],
                    help="dtype of the upstream gradients dY (the window sums are fp32 either way)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-tokens", type=int, default=0,
                    help="tokens per micro-step in the oracle's bounded sample (0 = all)")
    ap.add_argument("--cpu-windows", type=int, default=3,
                    help="windows in the oracle's bounded sample (at most --distinct-windows)")
    ap.add_argument("--distinct-windows", type=int, default=4,
                    help="distinct token windows cycled through (inputs stay resident)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only copy a 4 GiB fp32 tensor 3 times (the known-size kernel that scales "
                         "rocprofv3's FETCH_SIZE / WRITE_SIZE counters to bytes), then exit")
    ap.add_argument("--schedule", default="serial", choices=["serial", "overlap"],
                    help="burst modes: serial sorts each window inside its step; overlap keeps the "
                         "window's keys ahead and sorts them on a second stream while the forwards run "
                         "(ngram_window_keys / ngram_window_sort, NGRAM_OPT_PRESORT). With nothing but "
                         "the forwards to overlap, the sort slows them about as much as it saves. Spread "
                         "mode is always serial")
    ap.add_argument("--events-all", action="store_true",
                    help="HIP events on every launch of every kernel group (each event-carrying kernel "
                         "leaves the stream idle for a few microseconds; the default times the reduction "
                         "and sort of every window, one forward per window and the spread step)")
    ap.add_argument("--path", default="fused", choices=["fused", "accum"],
                    help="fused: the window's last micro-step goes through ngram_embed_bwd_step "
                         "(reduction fused with the step); accum: every micro-step through "
                         "ngram_embed_bwd_accum, then ngram_sparse_step")
    return ap.parse_args()


def workload(name):
    from sparse_hashed_gram_amd import workloads
    return {"tiny": workloads.TINY, "shard": workloads.SHARD, "full": workloads.FULL,
            "collision": workloads.COLLISION, "value": workloads.VALUE}[name]


def device_table(torch, R, dtype, seed, chunk=1 << 21):
    W = torch.empty((R, 768), dtype=dtype, device="cuda")
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    for s in range(0, R, chunk):
        e = min(R, s + chunk)
        W[s:e] = (torch.randn((e - s, 768), generator=g, device="cuda") * 0.02).to(dtype)
    return W


NEST_MIN_KEYS = 1 << 20   # the library's nested sort: reductions of at least this many keys


def nested_keys(torch, rb, rt, known=None, nest=True):
    """Trigram keys the fused reduction's bigram pass completes (so the
    trigram pass does not read their dY rows again): keys of trigram rows new
    to the window (not in `known`) whose keys lie in one 2,048-key tile of the
    trigram order and share one bigram row (nest), or that occur once (the
    singleton split alone, without the nested sort).  rb, rt: the rows of the
    positions, in stream order."""
    n = rb.numel()
    if n == 0:
        return 0
    if not nest:
        u, inv, cnt = torch.unique(rt, return_inverse=True, return_counts=True)
        single = cnt[inv] == 1
        if known is not None:
            single &= ~torch.isin(rt, known)
        return int(single.sum())
    idx = torch.arange(n, device=rb.device)
    ot = torch.sort(rt, stable=True).indices
    Rt = rt[ot]
    head = torch.ones(n, dtype=torch.bool, device=rb.device)
    head[1:] = Rt[1:] != Rt[:-1]
    end = torch.ones(n, dtype=torch.bool, device=rb.device)
    end[:-1] = Rt[1:] != Rt[:-1]
    hidx = torch.cummax(torch.where(head, idx, torch.zeros_like(idx)), 0).values
    eidx = torch.flip(torch.cummin(torch.flip(torch.where(end, idx, torch.full_like(idx, n)), [0]), 0).values, [0])
    seg = torch.cumsum(head.long(), 0) - 1
    bkey = rb[ot]
    bad = torch.zeros(n, dtype=torch.bool, device=rb.device)
    bad[1:] = (~head[1:]) & (bkey[1:] != bkey[:-1])
    if known is not None:
        bad |= head & torch.isin(Rt, known)
    fail = torch.zeros(int(seg[-1]) + 1, dtype=torch.int32, device=rb.device)
    fail.scatter_reduce_(0, seg, bad.int(), reduce="amax")
    nested = ((hidx // 2048) == (eidx // 2048)) & (fail[seg] == 0)
    return int(nested.sum())


def window_stats(torch, N, cfg, toks):
    """From the library's own hash, per micro-step and table in use: distinct
    rows, rows new to the window, and (trigram) the keys the fused reduction
    of that micro-step would complete in its bigram pass (nested_keys, rows
    already in the window excluded), and the rows that occur once in it;
    distinct rows of the whole window; the keys the window's fused reduction
    completes in its bigram pass.  A token-indexed table has one channel."""
    nch = 1 if cfg.options & N.OPT_DIRECT else 2
    steps = []
    seen = [None] * nch
    all_r = [[], []]
    for tok in toks:
        idx = N.hash(cfg, tok)
        per = []
        rows = [(idx[c] & 0x7FFFFFFF).long() for c in range(nch)]
        for c in range(nch):
            r = rows[c]
            u, cnt = torch.unique(r, return_counts=True)
            fresh = torch.ones_like(u, dtype=torch.bool) if seen[c] is None else ~torch.isin(u, seen[c])
            nest = bool(cfg.options & N.OPT_NEST_ALWAYS) or r.numel() >= NEST_MIN_KEYS
            handled = nested_keys(torch, rows[0], r, seen[1], nest) if c == 1 else 0
            single = int((cnt == 1).sum()) if c == 1 else 0
            per.append((int(u.numel()), int(fresh.sum()), handled, single))
            seen[c] = u if seen[c] is None else torch.unique(torch.cat([seen[c], u]))
            all_r[c].append(r)
        steps.append(per)
    handled_win = 0
    if nch == 2:
        rb_w, rt_w = torch.cat(all_r[0]), torch.cat(all_r[1])
        nest = bool(cfg.options & N.OPT_NEST_ALWAYS) or cfg.max_tokens * cfg.accum_steps >= NEST_MIN_KEYS
        handled_win = nested_keys(torch, rb_w, rt_w, None, nest)
    return steps, [int(s.numel()) for s in seen], handled_win


STATE = 8     # one (v, t_last) record per row


def algorithmic_bytes(T, stats, row_bytes, mode, path, dy_row=768 * 4, radix_passes=3):
    """Bytes each kernel group moves per window, listed per launch, two ways.

    "min": what the method itself cannot avoid moving.  A token's forward
      reads its two signed table rows and writes its output row (plus its
      id).  A reduction reads every upstream gradient row it is given once
      and the hashed row id of each position in each channel (4 B); a row it
      steps reads and writes its table row and its 8-byte state; in spread
      mode a micro-step's distinct rows also write (new to the window) or
      read and write (already there) their fp32 window row, and the fused
      last micro-step reads the window row of each row already there.  The
      separate step reads the window row, table row, state and slot id of
      each row left to it and writes the table row and state.
    "kernel": the dY rows the kernels actually read.  The bigram pass reads
      the dY row of every key.  The accumulating trigram pass reads those of
      keys whose row is not a singleton of the micro-step (a singleton is
      stored into the window by the bigram pass from the dY row it holds);
      the fused trigram pass reads those of keys whose row the bigram pass
      does not complete itself (nested_keys: singletons and nested runs new
      to the window), so the other trigram rows are read twice.  The other
      terms are as in "min".
    stash (burst): dY row read and written (copying), token id, two indices,
    row code.  dY rows count dy_row bytes (3,072 fp32, 1,536 bf16); window
    rows are fp32."""
    steps, uwin, handled_win = stats
    A = len(steps)
    nch = len(uwin)   # tables in use: 2, or 1 for a token-indexed table
    fwd = T * ((nch + 1) * row_bytes + 4)
    table_state = 2 * row_bytes + 2 * STATE
    step_row = ROW_F32 + table_state + 4
    ids = 4 * nch
    # sort: each radix pass reads and writes a (row, payload) pair per key of
    # every channel
    mn = {"fwd": [fwd] * A, "sort": [nch * T * 16 * radix_passes] * A}
    kn = {"fwd": [fwd] * A, "sort": [nch * T * 16 * radix_passes] * A}
    if mode in ("burst", "burst_ref"):
        n = A * T
        copy = 2 * dy_row if mode == "burst" else 0
        for d in (mn, kn):
            d["stash"] = [T * (copy + 4 + 8 + 4)] * A
            d["sort"] = [nch * n * 16 * radix_passes]
            d["step"] = [0]
        rows = sum(uwin) * table_state + n * ids
        mn["reduce"] = [n * dy_row + rows]
        kn["reduce"] = [(nch * n - handled_win) * dy_row + rows]
        return {"min": mn, "kernel": kn}
    red_m, red_k = [], []
    last = A - 1 if path == "fused" else A
    for m in range(last):
        win_rows = sum(new * ROW_F32 + (u - new) * 2 * ROW_F32 for (u, new, _, _) in steps[m])
        red_m.append(T * dy_row + win_rows + T * ids)
        red_k.append(sum((T - single) * dy_row for (_, _, _, single) in steps[m]) + win_rows + T * ids)
    fused_rows = 0
    if path == "fused":
        rows = sum((u - new) * ROW_F32 + u * table_state for (u, new, _, _) in steps[-1])
        red_m.append(T * dy_row + rows + T * ids)
        red_k.append(sum((T - handled) * dy_row for (_, _, handled, _) in steps[-1]) + rows + T * ids)
        fused_rows = sum(u for (u, _, _, _) in steps[-1])
    mn["reduce"], kn["reduce"] = red_m, red_k
    mn["step"] = kn["step"] = [(sum(uwin) - fused_rows) * step_row]
    return {"min": mn, "kernel": kn}


def code_text(src: str) -> str:
    """A C++ source's code alone: comments dropped, runs of whitespace made
    one space, so that a comment edit does not read as a kernel change.
    String and character literals are kept as written."""
    out, i, n = [], 0, len(src)
    while i < n:
        c = src[i]
        if c in "\"'":
            j = i + 1
            while j < n and src[j] != c:
                j += 2 if src[j] == "\\" else 1
            out.append(src[i:j + 1])
            i = j + 1
        elif src.startswith("//", i):
            j = src.find("\n", i)
            i = n if j < 0 else j
        elif src.startswith("/*", i):
            j = src.find("*/", i + 2)
            i = n if j < 0 else j + 2
        else:
            out.append(c)
            i += 1
    return " ".join("".join(out).split())


def src_hash(name):
    """Hash of a kernel source's code (comments and layout ignored): the key
    of its PMC summaries."""
    p = os.path.join(ROOT, "sparse_hashed_gram_amd", "csrc", name)
    with open(p, encoding="utf-8") as f:
        return hashlib.sha256(code_text(f.read()).encode()).hexdigest()[:16]


def pmc_traffic(group, workload_key, mode, dy_dtype):
    """HBM bytes per launch of a kernel group from a committed rocprofv3 PMC
    summary (profiles/pmc_*.md, FETCH_SIZE and WRITE_SIZE scaled by a plain
    copy's reading), if it was taken on the same workload, mode and dY dtype
    and on the kernel source as it is now; else None."""
    import glob
    want = src_hash(KERNEL_SRC[group])
    for p in sorted(glob.glob(os.path.join(ROOT, "profiles", "pmc_*.md"))):
        kv = {}
        with open(p) as f:
            for line in f:
                if ":" in line and not line.startswith(("#", "|", "rocprofv3")):
                    k, _, v = line.partition(":")
                    kv[k.strip()] = v.strip()
        if (kv.get("kernel") == group and kv.get("source_sha256_16") == want and kv.get("mode") == mode
                and kv.get("dy_dtype") == dy_dtype and kv.get("workload") == workload_key):
            try:
                return float(kv["hbm_bytes_per_launch"])
            except (KeyError, ValueError):
                return None
    return None


def host_info():
    """Core count, CPU model and RAM of the machine the oracle ran on."""
    info = {"nproc": os.cpu_count()}
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    info["cpu_model"] = line.split(":", 1)[1].strip()
                    break
        with open("/proc/meminfo") as f:
            for line in f:
                if line.startswith("MemTotal"):
                    info["ram_gib"] = round(int(line.split()[1]) / 2 ** 20, 1)
                    break
    except OSError:
        pass
    return info


def cpu_baseline(w, toks_np, T_sample, dys_fn):
    """The oracle on a bounded sample of the same workload: whole windows of
    4 micro-steps of T_sample tokens each (hash, forward, window gradient,
    sparse step on the touched rows), on all threads; then the first window
    at an eighth of the tokens on one thread.  Table rows are a snapshot of
    the rows a window touches; preparing inputs (dY, snapshots) is not
    timed."""
    import oracle
    el, ntok, n_upd = _oracle_windows(w, toks_np, T_sample, dys_fn)
    threads = oracle.threads()
    T1 = max(1, T_sample // 8)
    oracle.set_threads(1)
    try:
        el1, ntok1, _ = _oracle_windows(w, toks_np[:1], T1, dys_fn)
    finally:
        oracle.set_threads(threads)
    nw = len(toks_np)
    return {"value": ntok / el, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "seconds": el, "updated_rows_per_s": n_upd / el,
            "sample": (f"{nw} window(s) of 4 micro-steps x {T_sample} tokens of the same streams "
                       f"(hash, forward, window gradient, sparse step on {n_upd} touched rows in "
                       f"all; table rows as a snapshot of the touched rows)"),
            "one_thread": {"value": ntok1 / el1, "unit": "tokens/s", "seconds": el1,
                           "sample": f"the first window at 4 micro-steps x {T1} tokens, one thread"},
            "host": host_info()}


def _oracle_windows(w, toks_np, T_sample, dys_fn):
    import oracle
    el = 0.0
    ntok = 0
    n_upd = 0
    for win, wtoks in enumerate(toks_np):
        toks = [t[:T_sample] for t in wtoks]
        A = len(toks)
        dY = np.concatenate([dys_fn(win * A + m, T_sample) for m in range(A)])
        if w.direct:   # the token ids are the rows, every sign +1; no second table
            rows = [(t.astype(np.int64), np.zeros(len(t), np.uint8)) * 2 for t in toks]
        else:
            rows = [oracle.ngram_rows(t, w.vocab, w.eos_id, w.rows) for t in toks]
        nch = 1 if w.direct else 2
        rs = np.random.default_rng(win)
        ids = []
        snaps = []
        for c in range(2):
            u = np.unique(np.concatenate([r[2 * c] for r in rows]))
            ids.append(u)
            snaps.append(rs.integers(0x3C00, 0x3CFF, size=(len(u), 768)).astype(np.uint16)
                         ^ (rs.integers(0, 2, size=(len(u), 768)).astype(np.uint16) << 15))
        t0 = time.perf_counter()
        for m in range(A):
            if w.direct:   # the forward is a gather of the snapshot rows
                snaps[0][np.searchsorted(ids[0], toks[m])]
                continue
            rb, nb, rt, nt, _ = oracle.ngram_rows(toks[m], w.vocab, w.eos_id, w.rows)
            oracle.forward(snaps[0], snaps[1], rb, nb, rt, nt, ids_b=ids[0], ids_t=ids[1],
                           out_dtype="bf16")
        for c in range(nch):
            r = np.concatenate([x[2 * c] for x in rows])
            n = np.concatenate([x[2 * c + 1] for x in rows])
            touched, G = oracle.window_grad(r, n, dY)
            pos = np.searchsorted(ids[c], touched)
            oracle.sparse_step(G, snaps[c][pos], np.zeros(len(touched), np.float32),
                               np.zeros(len(touched), np.int32), 1, w.lr, w.beta2, w.eps)
            n_upd += len(touched)
        el += time.perf_counter() - t0
        ntok += sum(len(t) for t in toks)
        del dY, rows, snaps
    return el, ntok, n_upd


SSM_METRIC = "sampled-softmax loss tokens/s (forward + backward); achieved TFLOP/s vs bf16 matrix-core peak"
MFMA_BF16_PEAK_TFLOPS = 2500.0
SSM_GROUPS = ("cand", "fwd", "lse", "trans", "dz", "dx", "dw")


def cpu_baseline_ssm(batches, C, T_sample):
    """The sampled-softmax oracle (fp64 numpy) on a bounded sample: the first
    T_sample positions of each batch, all C candidates (candidate set, loss
    forward, backward)."""
    import oracle.ssm as orc
    el = 0.0
    n = 0
    for tgt, X, W, perm, g in batches:
        t, x, gg = tgt[:T_sample], X[:T_sample], g[:T_sample]
        t0 = time.perf_counter()
        cand, slot, _, ok = orc.candidates(t, perm, len(W), C)
        if not ok:
            continue
        orc.loss_fwd(x, W, cand, slot)
        orc.loss_bwd(x, W, cand, slot, gg)
        el += time.perf_counter() - t0
        n += len(t)
    threads = os.environ.get("OMP_NUM_THREADS") or str(os.cpu_count())
    return {"value": n / el if el else None, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "seconds": el, "host": host_info(),
            "sample": (f"{len(batches)} batch(es) x first {T_sample} positions, all {C} candidates "
                       f"(candidate set, fp64 loss forward and backward; numpy BLAS threads = {threads})")}


def main_ssm(args, torch):
    """One step = one micro-batch through the sampled-softmax loss: the
    candidate set, the forward (loss, lse) and the backward (dX, dW[S] +=).
    Inputs resident in HBM; a few distinct batches cycled."""
    from sparse_hashed_gram_amd import ssm as S
    from sparse_hashed_gram_amd import synth
    from sparse_hashed_gram_amd.hipevents import Event

    torch.cuda.set_device(0)
    V, T, C, D = 50304, args.ssm_tokens, args.candidates, 768
    nb = max(1, min(args.distinct_windows, 4))
    cfg = S.config(V, C, T)
    ws = S.Workspace(cfg)
    host = [synth.ssm_inputs(b, T, V) for b in range(nb)]
    W = torch.from_numpy(host[0][2]).to(torch.bfloat16).cuda()
    batches = []
    for tgt, X, _, perm, g in host:
        batches.append((torch.from_numpy(tgt).cuda(), torch.from_numpy(X).to(torch.bfloat16).cuda(),
                        torch.from_numpy(perm).cuda(), torch.from_numpy(g).cuda()))
    cand = torch.empty(C, dtype=torch.int32, device="cuda")
    slot = torch.empty(T, dtype=torch.int32, device="cuda")
    loss = torch.empty(T, dtype=torch.float32, device="cuda")
    lse = torch.empty(T, dtype=torch.float32, device="cuda")
    dX = torch.empty((T, D), dtype=torch.float32, device="cuda")
    dW = torch.zeros((V, D), dtype=torch.float32, device="cuda")

    def run(k, ev=None):
        if ev is not None:
            for gi, name in enumerate(SSM_GROUPS):
                a, b = Event(), Event()
                ev[name].append((a, b))
                S.profile_events(gi, a.handle, b.handle)
        tgt, X, perm, g = batches[k]
        S.candidates(cfg, ws, tgt, perm, cand, slot)
        S.loss_fwd(cfg, ws, X, W, cand, slot, loss, lse)
        S.loss_bwd(cfg, ws, X, W, cand, slot, lse, g, dW, dX)
        if ev is not None:
            for gi in range(S.PROF_GROUPS):
                S.profile_events(gi, None, None)

    for i in range(args.warmup):
        run(i % nb)
    torch.cuda.synchronize()
    ev = {n: [] for n in SSM_GROUPS}
    t0 = time.perf_counter()
    for i in range(args.steps):
        run(i % nb, ev)
    torch.cuda.synchronize()
    el = time.perf_counter() - t0
    flags = S.device_status(cfg, ws)
    if flags:
        print(f"bench.py: sampled-softmax device flags {flags:#x} set", file=sys.stderr)
        sys.exit(1)
    flop = 2.0 * T * C * D   # one contraction over the batch and the candidate set
    kflop = {"fwd": flop, "dx": flop, "dw": flop}
    # dz streams what the forward kept of its logits (fp16 exp(z - M)) and
    # writes dz in bf16, over the 128-padded batch and set
    Tq, Cq = -(-T // 128) * 128, -(-C // 128) * 128
    kbytes = {"dz": (2 + 2) * Tq * Cq}
    kernels = {}
    for name in SSM_GROUPS:
        ms_l = [a.elapsed_ms(b) for a, b in ev[name]]
        q1, med, q3 = (float(x) for x in np.percentile(ms_l, [25, 50, 75]))
        k = {"ms_per_launch": round(float(np.mean(ms_l)), 4), "ms_median": round(med, 4),
             "ms_iqr": round(q3 - q1, 4), "timed_launches": len(ms_l)}
        if name in kflop:
            tf = kflop[name] / (np.mean(ms_l) * 1e-3) / 1e12
            k.update({"flop_per_launch": kflop[name], "achieved_tflops": round(tf, 1),
                      "frac_of_mfma_peak": round(tf / MFMA_BF16_PEAK_TFLOPS, 4)})
        if name in kbytes:
            gbs = kbytes[name] / (np.mean(ms_l) * 1e-3) / 1e9
            k.update({"bytes_per_launch": kbytes[name], "achieved_gbs": round(gbs, 1),
                      "frac_of_hbm_peak": round(gbs / HBM_PEAK_GBPS, 4)})
        kernels[name] = k
    dom = max(kflop, key=lambda n: kernels[n]["ms_per_launch"])
    ms_step = el / args.steps * 1e3
    res = {
        "metric": SSM_METRIC,
        "value": round(T * args.steps / el, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic: Zipf next-token targets, N(0,1) hidden states, N(0,0.05) lm_head",
        "config": {"workload": f"sampled softmax: {T} positions x {C} candidates of a {V}-id vocabulary, "
                               f"dim {D}", "tokens_per_micro_step": T, "candidates": C, "vocab": V,
                   "dim": D},
        # the three contractions the method needs (forward, dX, dW)
        "path_tflops": round(3 * flop / (ms_step * 1e-3) / 1e12, 1),
        "kernels": kernels,
        "roofline": {"bound": "mfma", "kernel": dom, "achieved": kernels[dom]["achieved_tflops"],
                     "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": kernels[dom]["frac_of_mfma_peak"],
                     "traffic": pmc_traffic("ssm_" + dom, f"ssm_{T}x{C}", "ssm", "bf16")},
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        del ws, dW, dX, batches
        torch.cuda.empty_cache()
        Ts = args.cpu_tokens if args.cpu_tokens > 0 else 4096
        res["cpu_baseline"] = cpu_baseline_ssm(host[:2], C, min(T, Ts))
    print(json.dumps(res))


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py: this library runs on one GPU only (asked for --gpus {args.gpus}); the "
              "table lives whole on one MI355X and there is no multi-GPU path", file=sys.stderr)
        sys.exit(2)
    import torch

    if args.copy_calibration:
        n = 1 << 30   # 1 Gi floats = 4 GiB read and 4 GiB written per copy
        x = torch.ones(n, dtype=torch.float32, device="cuda")
        y = torch.empty_like(x)
        torch.cuda.synchronize()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
        ev[0].record()
        for k in range(3):
            y.copy_(x)
            ev[k + 1].record()
        torch.cuda.synchronize()
        ms = [ev[k].elapsed_time(ev[k + 1]) for k in range(3)]
        print(json.dumps({"copy_calibration_bytes_per_copy": 4 * n, "copies": 3, "ms_per_copy": ms,
                          "copy_gbps_read_plus_write": round(8 * n / (min(ms) * 1e-3) / 1e9, 1)}))
        return

    if args.workload == "ssm":
        return main_ssm(args, torch)

    from sparse_hashed_gram_amd import ngram as N
    from sparse_hashed_gram_amd import synth
    from sparse_hashed_gram_amd.hipevents import Event

    w = workload(args.workload)
    T = w.tokens_per_step
    A = w.accum_steps
    tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    row_bytes = ROW_BF16 if w.dtype == "bf16" else ROW_F32
    torch.cuda.set_device(0)
    overlap = args.schedule == "overlap" and args.mode in ("burst", "burst_ref")
    cfg = N.config(w.vocab, w.eos_id, w.rows, w.dtype, max_tokens=T, accum_steps=A, mode=args.mode,
                   dy_dtype=args.dy_dtype, presort=overlap, direct=w.direct)
    dy_row = 768 * (2 if args.dy_dtype == "bf16" else 4)

    nch = 1 if w.direct else 2   # a token-indexed table has no second table
    W = [device_table(torch, w.rows[c], tdt, 1000 + c) for c in range(nch)] + [None] * (2 - nch)
    state = [N.new_state(w.rows[c]) for c in range(nch)] + [None] * (2 - nch)
    ws = N.Workspace(cfg)
    out = torch.empty((T, 768), dtype=tdt, device="cuda")
    nwin = max(1, args.distinct_windows)
    toks_np = [[synth.tokens(w, win * A + m) for m in range(A)] for win in range(nwin)]
    toks = [[torch.from_numpy(t).cuda() for t in win] for win in toks_np]
    g = torch.Generator(device="cuda")
    g.manual_seed(7)
    dys = [torch.randn((T, 768), generator=g, device="cuda").to(cfg.dy_torch_dtype) for _ in range(A)]
    stats = [window_stats(torch, N, cfg, toks[k]) for k in range(nwin)]
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream().cuda_stream

    t_step = [0]
    burst = args.mode in ("burst", "burst_ref")
    gid = {"fwd": N.PROF_FWD, "sort": N.PROF_SORT, "reduce": N.PROF_REDUCE, "step": N.PROF_STEP,
           "stash": N.PROF_STASH}

    # Events ride on the timed kernels' own dispatches, but every kernel that
    # carries one still leaves the stream idle for a few microseconds around
    # it.  So they go on a sample of launches that covers every group's
    # launch kinds: the reduction and sort of every window (the dominant
    # kernels), one forward per window (micro-step i mod 4 in window i, so
    # every micro-step's forward is sampled equally), and the spread path's
    # step; --events-all times every launch of every group.
    def arm(ev, groups, win, m):
        if ev is None:
            return
        for grp in groups:
            if not args.events_all and (grp == "stash" or (grp == "fwd" and m != win % A)
                                        or (grp == "step" and burst)):
                continue
            a, b = Event(), Event()
            ev[grp].append((a, b, win, m))
            N.profile_events(gid[grp], a.handle, b.handle)

    def disarm():
        for k in range(N.PROF_GROUPS):
            N.profile_events(k, None, None)

    fused_last = args.path == "fused" and not burst
    main = torch.cuda.current_stream()
    side = torch.cuda.Stream()

    def run_window(k, ev=None, win=0):
        t_step[0] += 1
        if overlap:
            # the window's keys depend on its tokens only: keep them and sort
            # them on the side stream while the forwards run on the main one
            keys_done, sort_done = torch.cuda.Event(), torch.cuda.Event()
            side.wait_stream(main)
            with torch.cuda.stream(side):
                for m in range(A):
                    N.window_keys(cfg, ws, toks[k][m])
                keys_done.record(side)
                arm(ev, ("sort",), win, 0)
                N.window_sort(cfg, ws)
                disarm()
                sort_done.record(side)
        for m in range(A):
            arm(ev, ("fwd",), win, m)
            N.embed_fwd(cfg, W[0], W[1], toks[k][m], out=out)
            disarm()
            if overlap and m == 0:
                main.wait_event(keys_done)   # the backward only attaches dY to the kept keys
            if fused_last and m == A - 1:
                arm(ev, ("sort", "reduce", "step"), win, m)
                N.embed_bwd_step(cfg, ws, toks[k][m], dys[m], W[0], W[1], state[0], state[1], t_step[0],
                                 w.lr, w.beta2, w.eps)
                disarm()
                return
            arm(ev, ("stash",) if burst else ("sort", "reduce"), win, m)
            N.embed_bwd_accum(cfg, ws, toks[k][m], dys[m])
            disarm()
        if overlap:
            main.wait_event(sort_done)
        arm(ev, ("reduce", "step") if overlap else ("sort", "reduce", "step") if burst else ("step",), win,
            0 if burst else A)
        N.sparse_step(cfg, ws, W[0], W[1], state[0], state[1], t_step[0], w.lr, w.beta2, w.eps)
        disarm()

    for i in range(args.warmup):
        run_window(i % nwin)
    torch.cuda.synchronize()

    ev = {g_: [] for g_ in GROUPS}
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        run_window(i % nwin, ev, i)
    torch.cuda.synchronize()
    el = time.perf_counter() - t0
    flags = N.device_status(cfg, ws)
    if flags:
        print(f"bench.py: device flags {flags:#x} set", file=sys.stderr)
        sys.exit(1)

    used = [g_ for g_ in GROUPS if ev[g_]]
    timed_stats = [stats[i % nwin] for i in range(args.steps)]
    rbits = max(1, int(max(w.rows) - 1).bit_length())
    passes = (rbits + 8) // 9   # the library's 9-bit radix digits
    bytes_ = [algorithmic_bytes(T, s, row_bytes, args.mode, args.path, dy_row, passes) for s in timed_stats]
    ms_all = {g_: [a.elapsed_ms(b) for a, b, _, _ in ev[g_]] for g_ in used}

    def per_launch(kind):
        # bytes of each timed launch: launch m of the window's list (groups
        # with one launch per window have a one-entry list), then per group
        # all bytes of its timed launches over their number
        by = {g_: [bytes_[win][kind][g_][min(m, len(bytes_[win][kind][g_]) - 1)] for _, _, win, m in ev[g_]]
              for g_ in used}
        return {g_: float(np.sum(by[g_])) / len(ms_all[g_]) for g_ in used}

    per_step = {g_: len(bytes_[0]["min"][g_]) for g_ in used}
    ms = {g_: float(np.mean(ms_all[g_])) for g_ in used}
    abytes = per_launch("min")
    kbytes = per_launch("kernel")
    upd_rows = float(np.mean([sum(s[1]) for s in timed_stats]))
    total_ms = {g_: ms[g_] * per_step[g_] for g_ in used}
    dom = max([g_ for g_ in ("fwd", "reduce", "step") if g_ in used], key=lambda g_: total_ms[g_])
    if burst or args.path == "fused":
        # the step runs (partly) inside the last reduction launch
        last = [t for t, (_, _, _, m) in zip(ms_all["reduce"], ev["reduce"]) if burst or m == A - 1]
        step_ms_per_window = total_ms.get("step", 0.0) + float(np.mean(last))
    else:
        step_ms_per_window = total_ms["step"]
    # the forward's compulsory bytes: each distinct row of a micro-step read
    # once (repeats could come from the caches), every output row written
    comp_fwd = [sum(u[0] for u in timed_stats[win][0][m]) * row_bytes + T * (row_bytes + 4)
                for _, _, win, m in ev["fwd"]] if "fwd" in used else []
    kernels = {}
    for g_ in used:
        gbps = abytes[g_] / (ms[g_] * 1e-3) / 1e9
        q1, med, q3 = (float(x) for x in np.percentile(ms_all[g_], [25, 50, 75]))
        kernels[g_] = {"ms_per_launch": round(ms[g_], 4), "ms_median": round(med, 4),
                       "ms_iqr": round(q3 - q1, 4), "timed_launches": len(ms_all[g_]),
                       "launches_per_step": per_step[g_],
                       "ms_per_step": round(total_ms[g_], 4),
                       "algorithmic_bytes_per_launch": int(abytes[g_]),
                       "achieved_gbps": round(gbps, 1), "frac_of_hbm_peak": round(gbps / HBM_PEAK_GBPS, 4)}
        if kbytes[g_] != abytes[g_]:
            kg = kbytes[g_] / (ms[g_] * 1e-3) / 1e9
            kernels[g_].update({"kernel_read_bytes_per_launch": int(kbytes[g_]),
                                "kernel_read_frac_of_hbm_peak": round(kg / HBM_PEAK_GBPS, 4)})
        if g_ == "fwd" and comp_fwd:
            cb = float(np.mean(comp_fwd))
            kernels[g_]["compulsory_bytes_per_launch"] = int(cb)
            kernels[g_]["compulsory_frac_of_hbm_peak"] = round(cb / (ms[g_] * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4)
    traffic = pmc_traffic(dom, args.workload, args.mode, args.dy_dtype)
    achieved = abytes[dom] / (ms[dom] * 1e-3) / 1e9
    roof = {"bound": "hbm", "kernel": dom, "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS,
            "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4),
            "traffic": traffic}

    res = {
        "metric": METRIC,
        "value": round(A * T * args.steps / el, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(el / args.steps * 1e3, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": f"{w.dtype} table, {args.dy_dtype} dY, f32 sums",
        "data": "synthetic: Zipf token streams with EoS-aligned documents, N(0,1) upstream gradients",
        "config": {"workload": w.name, "table_rows": w.rows[0] + w.rows[1], "dim": 768,
                   "table_dtype": w.dtype, "tokens_per_micro_step": T, "accum_steps": A,
                   "mode": args.mode, "path": args.path, "dy_dtype": args.dy_dtype,
                   "schedule": "overlap" if overlap else "serial",
                   "global_batch": A * T},
        "fwd_tokens_per_s": round(T / (ms["fwd"] * 1e-3), 1),
        # rows stepped per second of the kernels that step them (the step, plus
        # the fused reduction when the step is fused into it)
        "updated_rows_per_s": round(upd_rows / (step_ms_per_window * 1e-3), 1),
        "updated_rows_per_step": int(upd_rows),
        "kernels": kernels,
        "roofline": roof,
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        del W, state, ws, out, dys
        torch.cuda.empty_cache()
        Ts = T if args.cpu_tokens <= 0 else min(T, args.cpu_tokens)
        nw = max(1, min(args.cpu_windows, len(toks_np)))
        res["cpu_baseline"] = cpu_baseline(w, toks_np[:nw], Ts, lambda m, n: synth.dY(w, m, n))
    print(json.dumps(res))


if __name__ == "__main__":
    main()
