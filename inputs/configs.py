"""The five seeded synthetic workloads of the Sep-Attention hot path.

This module holds sizes, parameters and seeds only. It contains none of the
method's arithmetic: no mask, no attention, no cache rule.

Symbols follow the SepLLM pages: a = initial-token count (SepCache
``init_cache_size``), n = neighbouring window (``*_local_window_size``),
s = separator-cache cap (``sep_cache_size``), w = local window
(``local_size``), p = past window, c = a+s+p+w (``cache_size``).

Separator sets:
  * the tiny config uses ids 0..7 in a 1000-id vocabulary;
  * the Llama-3-shaped configs use the Llama-3 separator ids that the SepLLM
    study notes list for the training-free configs
    (pengpengyi92.github.io "HKUDS047: SepLLM ...", section "Separator Tokens").
    The vocabulary bound 128256 is a choice made here; the pages do not state
    it, and any bound above 128000 yields identical separator flags.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Tuple

LLAMA3_SEP_IDS: Tuple[int, ...] = (13, 11, 30, 0, 26, 25, 198, 220, 128000)
LLAMA3_VOCAB = 128256
TINY_SEP_IDS: Tuple[int, ...] = tuple(range(8))
TINY_VOCAB = 1000


@dataclass(frozen=True)
class PrefillConfig:
    name: str
    B: int
    Hq: int
    Hkv: int
    D: int
    S: int
    dtype: str            # "f32" or "bf16"
    a: int
    n: int
    sep_ids: Tuple[int, ...]
    vocab: int
    p_sep: float          # i.i.d. separator probability (ignored for "runs")
    id_mode: str          # "iid" or "runs"
    run_mean: float       # mean segment length for "runs"
    seed: int


@dataclass(frozen=True)
class StreamConfig:
    name: str
    B: int
    Hq: int
    Hkv: int
    D: int
    dtype: str
    a: int
    s: int
    p: int
    w: int
    sep_ids: Tuple[int, ...]
    vocab: int
    p_sep: float
    history: int          # tokens ingested before the timed decode steps
    steps: int            # decode + cache-update steps
    pool: int             # distinct per-step q/k/v rows (stream uses pool[t mod pool])
    seed: int
    check_steps: int = 0  # steps compared with the oracle
    check_every: int = 0  # full cache-state check cadence (steps)

    @property
    def c(self) -> int:
        return self.a + self.s + self.p + self.w


TINY_PREFILL = PrefillConfig("tiny_prefill_f32_s512", B=1, Hq=2, Hkv=2, D=64, S=512, dtype="f32",
                   a=4, n=64, sep_ids=TINY_SEP_IDS, vocab=TINY_VOCAB, p_sep=0.1,
                   id_mode="iid", run_mean=0.0, seed=1001)

LLAMA3_LAYER_PREFILL = PrefillConfig("llama3_8b_layer_prefill_s8192", B=1, Hq=32, Hkv=8, D=128, S=8192,
                   dtype="bf16", a=4, n=256, sep_ids=LLAMA3_SEP_IDS, vocab=LLAMA3_VOCAB,
                   p_sep=0.12, id_mode="iid", run_mean=0.0, seed=1002)

STREAM_DECODE = StreamConfig("stream_decode_b1_4m_tokens", B=1, Hq=32, Hkv=8, D=128, dtype="bf16",
                  a=4, s=64, p=64, w=256, sep_ids=LLAMA3_SEP_IDS, vocab=LLAMA3_VOCAB,
                  p_sep=0.1, history=0, steps=4_194_304, pool=65_536, seed=1003,
                  check_steps=65_536, check_every=4096)

BATCHED_DECODE = StreamConfig("batched_decode_b64_h32768", B=64, Hq=32, Hkv=8, D=128, dtype="bf16",
                  a=4, s=256, p=28, w=512, sep_ids=LLAMA3_SEP_IDS, vocab=LLAMA3_VOCAB,
                  p_sep=0.12, history=32_768, steps=1024, pool=1024, seed=1004,
                  check_steps=1024, check_every=128)

LONG_PREFILL = PrefillConfig("long_prefill_runs_s131072", B=1, Hq=32, Hkv=8, D=128, S=131_072,
                   dtype="bf16", a=4, n=256, sep_ids=LLAMA3_SEP_IDS, vocab=LLAMA3_VOCAB,
                   p_sep=0.08, id_mode="runs", run_mean=12.0, seed=1005)

PREFILL_CONFIGS = {c.name: c for c in (TINY_PREFILL, LLAMA3_LAYER_PREFILL, LONG_PREFILL)}
STREAM_CONFIGS = {c.name: c for c in (STREAM_DECODE, BATCHED_DECODE)}
