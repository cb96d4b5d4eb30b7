"""The five synthetic workloads the path is measured and checked on.

Each workload mirrors the shapes of the hashed n-gram table in the NanoGPT
speedrun record: a vocabulary of 50,304 ids (agentic-affairs "NanoGPT
Training Record", benchmark definition section), a table of 84.6M rows split
between a bigram and a trigram channel (modded-nanogpt README, technique list;
agentic-affairs ablation section), 768 values per row (the quoted
@classiclarryd post gives one optimizer float per 768 parameters), updates
every 4 steps (same post; README technique list).  Token streams are synthetic
Zipf draws standing in for FineWeb text, which is not available here.

This module only holds sizes and knobs.  It contains none of the method's
arithmetic.
"""
from __future__ import annotations

import dataclasses

VOCAB = 50_304
EOS_ID = 50_256
DIM = 768


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    wid: int                 # seed namespace of this workload
    rows_bigram: int
    rows_trigram: int
    dtype: str               # "f32" or "bf16": table and forward-output type
    tokens_per_step: int     # T of one micro-step
    steps: int               # micro-steps generated for this workload
    accum_steps: int = 4
    zipf_s: float = 1.1
    hot_frac: float = 0.0    # share of tokens replaced by a draw from the hot set
    hot_size: int = 256
    doc_layout: str = "geometric"   # "fixed512" or "geometric"
    doc_mean: int = 1024
    doc_max: int = 2048
    lr: float = 0.01
    beta2: float = 0.95
    eps: float = 1e-8
    vocab: int = VOCAB
    eos_id: int = EOS_ID
    dim: int = DIM
    direct: bool = False     # one table indexed by the token id (value embeddings)

    @property
    def rows(self) -> tuple[int, int]:
        return (self.rows_bigram, self.rows_trigram)

    def table_bytes(self) -> int:
        el = 4 if self.dtype == "f32" else 2
        return (self.rows_bigram + self.rows_trigram) * self.dim * el


TINY = Workload(
    name="tiny: 2x4096x768 fp32 table, 8 micro-steps x 2048 tokens, EoS every 512",
    wid=1, rows_bigram=4096, rows_trigram=4096, dtype="f32",
    tokens_per_step=2048, steps=8, doc_layout="fixed512")

SHARD = Workload(
    name="one shard: 2x5,287,500x768 bf16, 49,152 tokens/step, Zipf 1.1, 64 steps",
    wid=2, rows_bigram=5_287_500, rows_trigram=5_287_500, dtype="bf16",
    tokens_per_step=49_152, steps=64)

FULL = Workload(
    name="full table: 2x42,300,000x768 bf16 (84.6M rows), 393,216 tokens/step, Zipf 1.1",
    wid=3, rows_bigram=42_300_000, rows_trigram=42_300_000, dtype="bf16",
    tokens_per_step=393_216, steps=8)

COLLISION = Workload(
    name="collision stress: 84.6M-row bf16 table, 393,216 tokens/step, Zipf 1.4 + 20% hot-256",
    wid=4, rows_bigram=42_300_000, rows_trigram=42_300_000, dtype="bf16",
    tokens_per_step=393_216, steps=8, zipf_s=1.4, hot_frac=0.2)

VALUE = Workload(
    name="value embeddings: token-indexed 50,304x768 bf16 table, 393,216 tokens/step, Zipf 1.1",
    wid=6, rows_bigram=VOCAB, rows_trigram=1, dtype="bf16",
    tokens_per_step=393_216, steps=8, direct=True)

SPREAD_BURST = Workload(
    name="spread vs burst: 84.6M-row bf16 table, 393,216 tokens/step, 32 steps",
    wid=5, rows_bigram=42_300_000, rows_trigram=42_300_000, dtype="bf16",
    tokens_per_step=393_216, steps=32)

ALL = (TINY, SHARD, FULL, COLLISION, SPREAD_BURST)
