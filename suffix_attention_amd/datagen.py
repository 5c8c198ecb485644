"""Seeded synthetic inputs (no arithmetic of the method lives here).

Values are i.i.d. N(0, 1) drawn in float32 by torch's generator and cast to the config's
dtype (bfloat16 rounds to nearest-even).  Seeds are 1_000_003 * cfg_id + tag with tags
  1: page permutation, 2: prompt K, 3: prompt V, 100 + 4 i + {0, 1, 2, 3}: member i's
  Q, response K, response V, dO.
A tensor's values depend on the generator's device: the same (seed, device) always gives
the same tensor, and callers that compare two implementations hand both the same tensor.
Device draws go in fixed chunks of 2^24 elements so that large tensors never need a
float32 copy in full.
"""
from __future__ import annotations

import torch

TAG_PERM, TAG_KP, TAG_VP = 1, 2, 3
CHUNK = 1 << 24


def seed(cfg_id: int, tag: int) -> int:
    return 1_000_003 * cfg_id + tag


def member_tag(i: int, which: str) -> int:
    return 100 + 4 * i + {"q": 0, "kr": 1, "vr": 2, "do": 3}[which]


def normal(shape, s: int, dtype=torch.float32, device="cpu") -> torch.Tensor:
    device = torch.device(device)
    g = torch.Generator(device=device)
    g.manual_seed(s)
    out = torch.empty(shape, dtype=dtype, device=device)
    flat = out.view(-1)
    n = flat.numel()
    for a in range(0, n, CHUNK):
        b = min(n, a + CHUNK)
        flat[a:b] = torch.randn(b - a, generator=g, dtype=torch.float32, device=device).to(dtype)
    return out


def page_table(n_pages: int, s: int, device="cpu") -> torch.Tensor:
    """table[logical page] = physical page: a seeded permutation of range(n_pages)."""
    g = torch.Generator()
    g.manual_seed(s)
    return torch.randperm(n_pages, generator=g).to(torch.int32).to(device)


def prefix_kv(cfg, device="cpu"):
    """Prompt keys and values in logical token order, [P, hkv, d] each."""
    shape = (cfg.P, cfg.hkv, cfg.d)
    return (normal(shape, seed(cfg.cfg_id, TAG_KP), cfg.dtype, device),
            normal(shape, seed(cfg.cfg_id, TAG_VP), cfg.dtype, device))


def member_inputs(cfg, i: int, device="cpu") -> dict:
    """Member i's query rows, response keys/values and upstream gradient."""
    sid = lambda w: seed(cfg.cfg_id, member_tag(i, w))  # noqa: E731
    return dict(
        q=normal((cfg.R, cfg.hq, cfg.d), sid("q"), cfg.dtype, device),
        kr=normal((cfg.R, cfg.hkv, cfg.d), sid("kr"), cfg.dtype, device),
        vr=normal((cfg.R, cfg.hkv, cfg.d), sid("vr"), cfg.dtype, device),
        do=normal((cfg.R, cfg.hq, cfg.d), sid("do"), cfg.dtype, device),
    )
