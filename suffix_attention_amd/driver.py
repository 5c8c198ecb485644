"""Serial group replay: G members, each replayed in reverse response blocks.

The prompt is captured once; members are then processed one after another (LongStraw
digest, "Method", step 3: rebuild one response graph, backpropagate, accumulate, free it,
then move to the next member).  Within a member, blocks of B response rows run from the
last to the first (explainer, "Two incompatible architectures": response blocks replayed in
reverse); block b sees the prompt and response keys [0, (b+1) B).  Prompt K/V gradient
pages are allocated at the first backward that touches them and written there, then
accumulated over blocks and members; everything a member allocates is released before the
next one, so peak memory does not grow with G (explainer, "Serial replay makes G a
schedule").
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Callable, Iterable

import torch

from . import api


@dataclass
class MemberResult:
    o: torch.Tensor | None
    lse: torch.Tensor | None
    dq: torch.Tensor | None
    dk_resp: torch.Tensor | None
    dv_resp: torch.Tensor | None
    peak_bytes: int
    base_bytes: int


@dataclass
class GroupReplay:
    """Accumulated state of one group: lazily allocated prompt gradient pages."""
    prefix: api.Prefix
    dk_pages: torch.Tensor | None = None
    dv_pages: torch.Tensor | None = None
    touched: list = field(default_factory=list)  # per shard: gradient pages already written

    def __post_init__(self):
        if not self.touched:
            self.touched = [False] * self.prefix.n_shards

    def _grad_pages(self):
        if self.dk_pages is None and self.prefix.prefix_len > 0:
            # allocated on first touch; the first backward writes every shard's pages
            self.dk_pages = torch.empty(self.prefix.k_pages.shape, dtype=torch.float32,
                                        device=self.prefix.k_pages.device)
            self.dv_pages = torch.empty_like(self.dk_pages)
        return self.dk_pages, self.dv_pages

    def replay_member(self, q, kr, vr, do, block: int, keep: str = "all",
                      on_block: Callable | None = None) -> MemberResult:
        """Forward + backward of one member's response, blocks in reverse order.

        keep: "all" returns o, lse, dq, dk_resp, dv_resp; "none" drops them at the end
        (the prompt gradient pages still accumulate)."""
        p = self.prefix
        R = q.shape[0]
        dev = q.device
        base = torch.cuda.memory_allocated(dev)
        torch.cuda.reset_peak_memory_stats(dev)
        o = torch.empty_like(q)
        lse = torch.empty((R, p.hq), dtype=torch.float32, device=dev)
        dq = torch.empty(q.shape, dtype=torch.float32, device=dev)
        dk_r = torch.empty(kr.shape, dtype=torch.float32, device=dev)
        dv_r = torch.empty(kr.shape, dtype=torch.float32, device=dev)
        dk_p, dv_p = self._grad_pages()
        nb = (R + block - 1) // block
        rows0 = min(block, R)
        ws_f = torch.empty((api.fwd_workspace_bytes(p, rows0) + 3) // 4, dtype=torch.float32, device=dev)
        ws_b = torch.empty((max(4, api.bwd_workspace_bytes(p, rows0)) + 3) // 4, dtype=torch.float32,
                           device=dev)
        for b in reversed(range(nb)):
            a, e = b * block, min(R, (b + 1) * block)
            api.replay_fwd(p, q[a:e], a, kr, vr, workspace=ws_f, o=o[a:e], lse=lse[a:e])
            first = [not t for t in self.touched]
            api.replay_bwd(p, q[a:e], a, kr, vr, o[a:e], lse[a:e], do[a:e], dk_r, dv_r, b == nb - 1, dk_p, dv_p,
                           shard_first_touch=first, workspace=ws_b, dq=dq[a:e])
            self.touched = [True] * p.n_shards
            if on_block is not None:
                on_block(b)
        del ws_f, ws_b
        peak = torch.cuda.max_memory_allocated(dev)
        if keep == "none":
            del o, lse, dq, dk_r, dv_r
            return MemberResult(None, None, None, None, None, peak, base)
        return MemberResult(o, lse, dq, dk_r, dv_r, peak, base)


def replay_group(prefix: api.Prefix, members: Iterable, block: int, keep: str = "all",
                 on_member: Callable | None = None) -> tuple[GroupReplay, list[MemberResult]]:
    """Replay every member serially.  `members` yields dicts with q, kr, vr, do (device
    tensors), or callables returning one, so inputs can be produced one member at a time."""
    grp = GroupReplay(prefix)
    results = []
    for i, m in enumerate(members):
        inp = m() if callable(m) else m
        r = grp.replay_member(inp["q"], inp["kr"], inp["vr"], inp["do"], block, keep=keep)
        del inp
        if on_member is not None:
            on_member(i, r)
        results.append(r)
    return grp, results
