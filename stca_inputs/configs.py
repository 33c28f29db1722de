"""Workload shapes (sizes, length mixes, targets per request)."""
from __future__ import annotations

import dataclasses
from dataclasses import dataclass


@dataclass(frozen=True)
class Config:
    key: str
    description: str
    n_users: int
    d: int
    h: int
    M: int
    r: int
    dtype: str                 # "f32" or "bf16" storage
    length: tuple              # ("fixed", L) | ("lognormal", median, mean, lo, hi)
    targets: tuple             # ("fixed", m) | ("1+poisson", lam)
    dup_prob: float = 0.0      # probability a history token repeats an earlier one
    dup_window: int = 3        # how far back a repeat may reach
    seed: int = 0

    @property
    def d_h(self) -> int:
        return self.d // self.h


CONFIGS = {
    c.key: c
    for c in [
        Config("tiny", "1 user, L=256, 4 targets, d=64, h=4, M=1, r=2, fp32",
               n_users=1, d=64, h=4, M=1, r=2, dtype="f32",
               length=("fixed", 256), targets=("fixed", 4)),
        Config("uniform", "256 users x L=2048, 8 targets/user, d=128, h=8, M=2, r=2, bf16",
               n_users=256, d=128, h=8, M=2, r=2, dtype="bf16",
               length=("fixed", 2048), targets=("fixed", 8)),
        Config("ragged", "512 users, L log-normal(median 1500) in [64,10000], 1+Poisson(5) targets, "
               "d=256, h=8, M=3, r=4, bf16",
               n_users=512, d=256, h=8, M=3, r=4, dtype="bf16",
               length=("lognormal", 1500.0, 2000.0, 64, 10000), targets=("1+poisson", 5.0)),
        Config("dense10k", "1024 users x L=10000, 16 targets/user, d=256, h=8, M=3, r=4, bf16, "
               "~10% same-ID repeats within 3 positions",
               n_users=1024, d=256, h=8, M=3, r=4, dtype="bf16",
               length=("fixed", 10000), targets=("fixed", 16), dup_prob=0.10, dup_window=3),
        Config("stress20k", "256 users x L=20000, 32 targets/user, d=512, h=16, M=4, r=4, bf16",
               n_users=256, d=512, h=16, M=4, r=4, dtype="bf16",
               length=("fixed", 20000), targets=("fixed", 32)),
    ]
}


def get_config(key: str) -> Config:
    try:
        return CONFIGS[key]
    except KeyError:
        raise KeyError(f"unknown workload {key!r}; known: {sorted(CONFIGS)}") from None


def scaled(cfg: Config, **changes) -> Config:
    """A copy of ``cfg`` with some fields replaced (e.g. fewer users for a quick test)."""
    return dataclasses.replace(cfg, **changes)
