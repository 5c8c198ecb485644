"""Named workloads of the replay-attention path and the work they count.

Each config is one layer of exact attention: a prompt of P tokens in 64-token pages with a
permuted page table, split into S contiguous page-shards, and G group members whose
responses of R tokens are replayed serially in reverse blocks of B rows.
"""
from __future__ import annotations

from dataclasses import dataclass

import torch


@dataclass(frozen=True)
class Config:
    name: str
    cfg_id: int
    P: int            # prompt tokens
    R: int            # response tokens per member
    B: int            # response rows per replayed block
    hq: int
    hkv: int
    d: int
    dtype: torch.dtype
    S: int            # prompt shards
    G: int            # group members

    @property
    def n_pages(self) -> int:
        return (self.P + 63) // 64

    @property
    def n_blocks(self) -> int:
        return (self.R + self.B - 1) // self.B

    @property
    def g(self) -> int:
        return self.hq // self.hkv

    def with_(self, **kw) -> "Config":
        d = dict(self.__dict__)
        d.update(kw)
        return Config(**d)


CONFIGS = {
    "tiny": Config("tiny", 0, P=4096, R=256, B=256, hq=4, hkv=1, d=64, dtype=torch.float32, S=2, G=1),
    "c128k": Config("c128k", 1, P=131072, R=1024, B=1024, hq=24, hkv=4, d=256, dtype=torch.bfloat16, S=8, G=2),
    "c1m": Config("c1m", 2, P=1048576, R=2048, B=512, hq=24, hkv=4, d=256, dtype=torch.bfloat16, S=8, G=8),
    "c2m": Config("c2m", 3, P=2097152, R=4096, B=1024, hq=24, hkv=4, d=256, dtype=torch.bfloat16, S=8, G=8),
    "stress": Config("stress", 4, P=4194304, R=262144, B=8192, hq=24, hkv=4, d=256, dtype=torch.bfloat16, S=16,
                     G=1),
    # prefix reuse: consecutive G = 8 optimizer cycles over one capture of 4,456,448 positions
    "reuse4m": Config("reuse4m", 5, P=4456448, R=4096, B=1024, hq=24, hkv=4, d=256, dtype=torch.bfloat16, S=8,
                      G=8),
}


def pairs(n_rows: int, q_start: int, P: int) -> int:
    """Visible (row, key) pairs per query head: every prompt key plus the causal response keys."""
    return n_rows * P + n_rows * q_start + n_rows * (n_rows + 1) // 2


def counted_flops(n_rows: int, q_start: int, P: int, hq: int, d: int) -> int:
    """Counted work of one forward + backward: per visible pair and head, 2 flops for each of
    4 multiply-add units forward (S, PV) and 10 backward (S, dP, dV, dQ, dK)."""
    return 14 * hq * d * pairs(n_rows, q_start, P)


def member_flops(cfg: Config) -> int:
    return counted_flops(cfg.R, 0, cfg.P, cfg.hq, cfg.d)
