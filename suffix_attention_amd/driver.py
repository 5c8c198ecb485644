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
                      on_block: Callable | None = None, store_ds: bool | None = None,
                      ds_budget: int | None = None) -> MemberResult:
        """Forward + backward of one member's response, blocks in reverse order.

        keep: "all" returns o, lse, dq, dk_resp, dv_resp; "none" drops them at the end
        (the prompt gradient pages still accumulate).  store_ds: give the backward the
        workspace in which it keeps dS for the dQ pass (True), or not (False); None does so
        when it fits in device memory (or in ds_budget bytes, if given), for all kv heads at
        once or for an equal chunk of them at a time."""
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
        nb_ws = api.bwd_workspace_bytes(p, rows0)
        if store_ds is not False and p.dtype == torch.bfloat16:
            # the first block replayed (the last) sees the most response keys: its size serves
            # all; without room for every kv head's dS, the largest number of kv heads dividing
            # hkv (equal chunks) whose dS fits
            nb_ds = api.bwd_ds_workspace_bytes(p, rows0, R)
            if store_ds or api.ds_fits(nb_ds, dev, budget=ds_budget):
                nb_ws = nb_ds
            else:
                for k in range(p.hkv - 1, 0, -1):
                    nb_k = api.bwd_ds_workspace_bytes(p, rows0, R, heads=k)
                    if p.hkv % k == 0 and api.ds_fits(nb_k, dev, budget=ds_budget):
                        nb_ws = nb_k
                        break
        ws_b = torch.empty((max(4, nb_ws) + 3) // 4, dtype=torch.float32, device=dev)
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
                 on_member: Callable | None = None, store_ds: bool | None = None,
                 ds_budget: int | None = None) -> tuple[GroupReplay, list[MemberResult]]:
    """Replay every member serially.  `members` yields dicts with q, kr, vr, do (device
    tensors), or callables returning one, so inputs can be produced one member at a time."""
    grp = GroupReplay(prefix)
    results = []
    for i, m in enumerate(members):
        inp = m() if callable(m) else m
        r = grp.replay_member(inp["q"], inp["kr"], inp["vr"], inp["do"], block, keep=keep, store_ds=store_ds,
                              ds_budget=ds_budget)
        del inp
        if on_member is not None:
            on_member(i, r)
        results.append(r)
    return grp, results


def prefill_capture(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, page_table: torch.Tensor, n_phys: int,
                    chunk: int, n_shards: int = 1, keep_o: bool = True):
    """Capture-side prefill without gradients: the prompt's own causal attention, chunk by chunk
    (digest, "Method", step 1: the prompt is evaluated once without autograd and its KV pages are
    retained).  Chunk [a, e) attends to the pages captured so far (tokens [0, a), split into
    n_shards page ranges) plus itself under the causal mask -- exactly a replay forward with the
    chunk as the "response" at q_start = 0 -- and its keys and values are then written into the
    pools.  q [P, hq, d], k / v [P, hkv, d]; chunk is a multiple of the page size.

    Returns (prefix over the whole prompt with n_shards shards, o [P, hq, d] or None, lse
    [P, hq] or None)."""
    if chunk <= 0 or chunk % api.PAGE:
        raise ValueError(f"chunk={chunk} must be a positive multiple of {api.PAGE}")
    P, hq, d = q.shape
    hkv = k.shape[1]
    dev = q.device
    k_pages = torch.zeros((n_phys, hkv, api.PAGE, d), dtype=k.dtype, device=dev)
    v_pages = torch.zeros_like(k_pages)
    o = torch.empty_like(q) if keep_o else None
    lse = torch.empty((P, hq), dtype=torch.float32, device=dev) if keep_o else None
    ws = None
    for a in range(0, P, chunk):
        e = min(P, a + chunk)
        pre = api.Prefix(hq, hkv, d, q.dtype, a, page_table, k_pages, v_pages,
                         api.even_shard_bounds(api.n_logical_pages(a), n_shards))
        need = api.fwd_workspace_bytes(pre, e - a)
        if ws is None or ws.numel() * ws.element_size() < need:
            ws = torch.empty(((need + 15) // 16) * 4, dtype=torch.float32, device=dev)
        oc, lc, _ = api.replay_fwd(pre, q[a:e], 0, k[a:e], v[a:e], workspace=ws,
                                   o=o[a:e] if keep_o else None, lse=lse[a:e] if keep_o else None)
        api.capture_pages(k[a:e], v[a:e], page_table, n_phys, first_tok=a, k_pages=k_pages, v_pages=v_pages)
    full = api.Prefix(hq, hkv, d, q.dtype, P, page_table, k_pages, v_pages,
                      api.even_shard_bounds(api.n_logical_pages(P), n_shards))
    return full, o, lse
