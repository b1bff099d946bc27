"""The five synthetic workload shapes.

Each one mirrors a model and context length the SpeCache summary evaluates
(LLaMA-3-8B at 8K, Mistral-7B-Instruct-v0.2 at 32K, §4 "experimental setup"),
with the 1-bit / 2-bit KIVI-style cache of §3 and the top-k of §4 (top-64 there;
1% of the context here, following the top-1% transfer study of §2, Figure 2).
The synthetic structure stands in for the pages' datasets (LongBench, PG19,
Needle-in-a-Haystack), none of which is used:

* keys ~ N(0,1) with a few outlier channels (the reason keys are quantized
  per channel, SemKV §2.1), or lognormal per-channel scales for the long case;
* values and queries ~ N(0,1);
* a planted peak: 0.5% of positions aligned with the query so that they carry
  about 90% of the attention mass (the sparsity observation of SpeCache §2).

`peak` is the logit strength of the planted positions (a dimensionless number
in units of scaled logits); it was chosen by tests/golden/calibrate_peak.py.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, replace


@dataclass(frozen=True)
class WorkloadConfig:
    name: str
    batch: int
    n_q_heads: int
    n_kv_heads: int
    seq_len: int
    head_dim: int
    bits: int
    top_k: int
    n_tokens: int = 2          # real token T_t and speculative token T'_{t+1}
    group: int = 32
    n_outlier: int = 0         # outlier key channels per KV head
    outlier_scale: float = 1.0
    lognormal_keys: bool = False
    peak: float | None = None  # planted-peak logit strength (None: no peak)
    peak_frac: float = 0.005   # fraction of positions planted
    n_layers: int = 1
    tail_len: int = 0
    seed: int = 0

    @property
    def gqa(self) -> int:
        return self.n_q_heads // self.n_kv_heads

    @property
    def n_planted(self) -> int:
        return int(math.ceil(self.peak_frac * self.seq_len)) if self.peak is not None else 0

    @property
    def sm_scale(self) -> float:
        return 1.0 / math.sqrt(self.head_dim)

    def with_(self, **kw) -> "WorkloadConfig":
        return replace(self, **kw)


CONFIGS = {
    "tiny": WorkloadConfig(
        name="tiny", batch=1, n_q_heads=4, n_kv_heads=2, seq_len=512, head_dim=64,
        bits=1, top_k=16, n_outlier=4, outlier_scale=8.0),
    "llama8k": WorkloadConfig(
        name="llama8k", batch=1, n_q_heads=32, n_kv_heads=8, seq_len=8192, head_dim=128,
        bits=2, top_k=64, n_outlier=8, outlier_scale=10.0, peak=11.87),
    "mistral32k": WorkloadConfig(
        name="mistral32k", batch=8, n_q_heads=32, n_kv_heads=8, seq_len=32768, head_dim=128,
        bits=1, top_k=328, n_outlier=8, outlier_scale=10.0, peak=11.38),
    "layers32": WorkloadConfig(
        name="layers32", batch=16, n_q_heads=32, n_kv_heads=8, seq_len=32768, head_dim=128,
        bits=1, top_k=328, n_outlier=8, outlier_scale=10.0, peak=11.38, n_layers=32),
    "long128k": WorkloadConfig(
        name="long128k", batch=4, n_q_heads=32, n_kv_heads=8, seq_len=131072, head_dim=128,
        bits=1, top_k=1024, lognormal_keys=True),
}


def get_config(name: str) -> WorkloadConfig:
    try:
        return CONFIGS[name]
    except KeyError:
        raise KeyError(f"unknown workload {name!r}; known: {sorted(CONFIGS)}") from None
