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
from .trace import trace_range


@dataclass(frozen=True)
class BwdPlan:
    """How a group's backward runs, fixed once for the whole group: the stored-dS pass in chunks
    of `heads` kv heads by `parts` consecutive key parts (the shards, then the response keys), or
    the recomputing dQ pass (heads == 0)."""
    heads: int
    parts: int

    @property
    def store_ds(self) -> bool:
        return self.heads > 0

    def describe(self, prefix: api.Prefix) -> str:
        if not self.store_ds:
            return "recompute"
        if self.heads == prefix.hkv and self.parts == prefix.n_shards + 1:
            return "stored dS"
        return f"stored dS in chunks of {self.heads} kv head(s) x {self.parts} key part(s)"


@dataclass
class MemberResult:
    o: torch.Tensor | None
    lse: torch.Tensor | None
    dq: torch.Tensor | None
    dk_resp: torch.Tensor | None
    dv_resp: torch.Tensor | None
    peak_bytes: int | None     # peak device memory while the member ran (track_peak), else None
    base_bytes: int            # device memory allocated when the member started
    plan: BwdPlan | None = None
    ws_bytes: int = 0          # bytes of the member's backward workspace


def _blocks(R: int, block: int):
    """Response row ranges [a, e) of the reverse replay order: last block first."""
    nb = (R + block - 1) // block
    return [(b * block, min(R, (b + 1) * block)) for b in reversed(range(nb))]


@dataclass
class GroupReplay:
    """Accumulated state of one group: lazily allocated prompt gradient pages, and the backward
    plan, chosen at the group's first member and kept for every member after it.

    store_ds: True forces the stored-dS backward over all keys at once, False the recomputing
    one; None picks the first of (all kv heads at once; equal chunks of kv heads, largest
    first; one kv head by the largest number of key parts) whose workspace fits in ds_budget
    bytes, or in 90% of what the device has free at the first member, else recomputes.
    track_peak: record each member's peak device memory (this resets torch's peak counter at
    each member's start); peak_bytes is then the largest over the group's members.
    check_owners: a debug run: every backward counts its writers (api.OwnerCounts) and the
    driver raises if a gradient half-page or a dQ part row had two (one host sync per block).
    fused: each block runs the fused forward + dQ pass (replay_fwd_dq, dO known before the
    forward) and then the backward without dQ (recomputing, no stored dS; bf16 only).
    Members, blocks and each block's forward and backward are roctx ranges (trace.py)."""
    prefix: api.Prefix
    store_ds: bool | None = None
    ds_budget: int | None = None
    track_peak: bool = False
    dk_pages: torch.Tensor | None = None
    dv_pages: torch.Tensor | None = None
    touched: list = field(default_factory=list)  # per shard: gradient pages already written
    plan: BwdPlan | None = None
    peak_bytes: int = 0
    check_owners: bool = False
    members_done: int = 0
    fused: bool = False

    def __post_init__(self):
        if not self.touched:
            self.touched = [False] * self.prefix.n_shards
        if self.fused and self.check_owners:
            raise ValueError("writer counting covers backward calls that form dQ; the fused step forms it earlier")

    def _grad_pages(self):
        if self.dk_pages is None and self.prefix.prefix_len > 0:
            # allocated at the first backward; it writes every shard's pages (first touch)
            self.dk_pages = torch.empty(self.prefix.k_pages.shape, dtype=torch.float32,
                                        device=self.prefix.k_pages.device)
            self.dv_pages = torch.empty_like(self.dk_pages)
        return self.dk_pages, self.dv_pages

    def _ws_bytes(self, plan: BwdPlan, n: int, key_end: int) -> int:
        p = self.prefix
        if not plan.store_ds:
            return api.bwd_workspace_bytes(p, n)
        return api.bwd_ds_workspace_bytes(p, n, key_end, heads=plan.heads, parts=plan.parts)

    def _choose_plan(self, blocks, dev) -> BwdPlan:
        p = self.prefix
        n_all = p.n_shards + 1
        if self.store_ds is False or p.dtype != torch.bfloat16 or self.fused:
            return BwdPlan(0, 0)
        cands = [BwdPlan(p.hkv, n_all)]
        cands += [BwdPlan(h, n_all) for h in range(p.hkv - 1, 0, -1) if p.hkv % h == 0]
        cands += [BwdPlan(1, k) for k in range(n_all - 1, 0, -1)]
        if self.store_ds:
            return cands[0]
        for c in cands:
            need = max(self._ws_bytes(c, e - a, e) for a, e in blocks)
            if api.ds_fits(need, dev, budget=self.ds_budget):
                return c
        return BwdPlan(0, 0)

    def replay_member(self, q, kr, vr, do, block: int, keep: str = "all",
                      on_block: Callable | None = None) -> MemberResult:
        """Forward + backward of one member's response, blocks in reverse order.

        keep: "all" returns o, lse, dq, dk_resp, dv_resp; "none" drops them at the end
        (the prompt gradient pages still accumulate)."""
        with trace_range(f"member {self.members_done}"):
            r = self._replay_member(q, kr, vr, do, block, keep, on_block)
        self.members_done += 1
        return r

    def _backward(self, args, kwargs, n: int, key_end: int, dev, where: str):
        if not self.check_owners:
            api.replay_bwd(*args, **kwargs)
            return
        with api.OwnerCounts(api.owner_slots(self.prefix, n, key_end), dev) as oc:
            api.replay_bwd(*args, **kwargs)
        oc.check(where)

    def _replay_member(self, q, kr, vr, do, block: int, keep: str, on_block: Callable | None) -> MemberResult:
        p = self.prefix
        R = q.shape[0]
        dev = q.device
        base = torch.cuda.memory_allocated(dev)
        if self.track_peak:
            torch.cuda.reset_peak_memory_stats(dev)
        o = torch.empty_like(q)
        lse = torch.empty((R, p.hq), dtype=torch.float32, device=dev)
        dq = torch.empty(q.shape, dtype=torch.float32, device=dev)
        dk_r = torch.empty(kr.shape, dtype=torch.float32, device=dev)
        dv_r = torch.empty(kr.shape, dtype=torch.float32, device=dev)
        blocks = _blocks(R, block)
        rows0 = max((e - a for a, e in blocks), default=0)
        f_bytes = api.fwd_dq_workspace_bytes(p, rows0) if self.fused else api.fwd_workspace_bytes(p, rows0)
        ws_f = torch.empty((f_bytes + 3) // 4, dtype=torch.float32, device=dev)
        ws_b = None
        for i, (a, e) in enumerate(blocks):
            with trace_range(f"block [{a}, {e}) forward"):
                if self.fused:
                    api.replay_fwd_dq(p, q[a:e], a, kr, vr, do[a:e], workspace=ws_f, o=o[a:e], lse=lse[a:e],
                                      dq=dq[a:e])
                else:
                    api.replay_fwd(p, q[a:e], a, kr, vr, workspace=ws_f, o=o[a:e], lse=lse[a:e])
            if ws_b is None:
                # the first backward: gradient pages (once per group), the plan (once per group),
                # and this member's workspace, sized for the largest of its blocks
                dk_p, dv_p = self._grad_pages()
                if self.plan is None:
                    self.plan = self._choose_plan(blocks, dev)
                ws_max = max(self._ws_bytes(self.plan, ee - aa, ee) for aa, ee in blocks)
                ws_b = torch.empty((max(4, ws_max) + 3) // 4, dtype=torch.float32, device=dev)
            # the workspace view is sized for this block exactly, so every block runs the plan
            nbytes = self._ws_bytes(self.plan, e - a, e)
            first = [not t for t in self.touched]
            with trace_range(f"block [{a}, {e}) backward"):
                kw = dict(shard_first_touch=first, workspace=ws_b[:(max(4, nbytes) + 3) // 4])
                kw.update(dq_pass=False) if self.fused else kw.update(dq=dq[a:e])
                self._backward((p, q[a:e], a, kr, vr, o[a:e], lse[a:e], do[a:e], dk_r, dv_r, i == 0, dk_p, dv_p),
                               kw, e - a, e, dev, f"member {self.members_done} block [{a}, {e})")
            self.touched = [True] * p.n_shards
            if on_block is not None:
                on_block((a, e))
        ws_bytes = 0 if ws_b is None else ws_b.numel() * 4
        del ws_f, ws_b
        peak = None
        if self.track_peak:
            peak = torch.cuda.max_memory_allocated(dev)
            self.peak_bytes = max(self.peak_bytes, peak)
        if keep == "none":
            del o, lse, dq, dk_r, dv_r
            return MemberResult(None, None, None, None, None, peak, base, self.plan, ws_bytes)
        return MemberResult(o, lse, dq, dk_r, dv_r, peak, base, self.plan, ws_bytes)


def replay_group(prefix: api.Prefix, members: Iterable, block: int, keep: str = "all",
                 on_member: Callable | None = None, store_ds: bool | None = None,
                 ds_budget: int | None = None, track_peak: bool = False,
                 check_owners: bool = False, fused: bool = False) -> tuple[GroupReplay, list[MemberResult]]:
    """Replay every member serially.  `members` yields dicts with q, kr, vr, do (device
    tensors), or callables returning one, so inputs can be produced one member at a time.
    store_ds, ds_budget, track_peak, check_owners and fused as for GroupReplay."""
    grp = GroupReplay(prefix, store_ds=store_ds, ds_budget=ds_budget, track_peak=track_peak,
                      check_owners=check_owners, fused=fused)
    results = []
    for i, m in enumerate(members):
        inp = m() if callable(m) else m
        r = grp.replay_member(inp["q"], inp["kr"], inp["vr"], inp["do"], block, keep=keep)
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
    api.check_page_table(page_table, n_phys)
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
        api.capture_pages(k[a:e], v[a:e], page_table, n_phys, first_tok=a, k_pages=k_pages, v_pages=v_pages,
                          check_table=False)
    full = api.Prefix(hq, hkv, d, q.dtype, P, page_table, k_pages, v_pages,
                      api.even_shard_bounds(api.n_logical_pages(P), n_shards))
    return full, o, lse
