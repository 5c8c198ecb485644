"""Python binding of the replay-attention C ABI (include/longstraw.h).

Argument marshalling only: shapes and dtypes are checked, device pointers and torch's
current HIP stream are passed through, and every step runs in the library's kernels.  torch
supplies device memory (outputs and workspaces are allocated here as torch tensors, so the
caching allocator owns them) and streams.
"""
from __future__ import annotations

import ctypes as C
import math
from dataclasses import dataclass, field

import torch

from . import _lib
from ._lib import LS_DTYPE_BF16, LS_DTYPE_F32, LongStrawError, check, lib

PAGE = 64

_DT = {torch.float32: LS_DTYPE_F32, torch.bfloat16: LS_DTYPE_BF16}


def _dtype_code(t: torch.dtype) -> int:
    if t not in _DT:
        raise LongStrawError(_lib.LS_ERR_UNSUPPORTED, f"dtype {t} (only float32 and bfloat16)")
    return _DT[t]


def _ptr(t):
    return None if t is None else C.c_void_p(t.data_ptr())


def _stream():
    return C.c_void_p(torch.cuda.current_stream().cuda_stream)


def _dev(t: torch.Tensor, name: str, dtype=None, shape=None):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    return t


def n_logical_pages(n_tok: int) -> int:
    return (n_tok + PAGE - 1) // PAGE


def even_shard_bounds(n_pages: int, n_shards: int) -> list[int]:
    """Contiguous logical page ranges [floor(s n / S), floor((s+1) n / S))."""
    return [(s * n_pages) // n_shards for s in range(n_shards + 1)]


@dataclass
class Prefix:
    """A captured prompt: paged K/V pools, the page table and the shard split."""
    hq: int
    hkv: int
    d: int
    dtype: torch.dtype
    prefix_len: int
    page_table: torch.Tensor          # int32 [n_logical_pages] on device
    k_pages: torch.Tensor             # [n_phys, hkv, 64, d]
    v_pages: torch.Tensor
    shard_bounds: list = field(default_factory=list)
    softmax_scale: float | None = None

    def __post_init__(self):
        if self.softmax_scale is None:
            self.softmax_scale = 1.0 / math.sqrt(self.d)
        if not self.shard_bounds:
            self.shard_bounds = even_shard_bounds(n_logical_pages(self.prefix_len), 1)
        self._bounds = (C.c_int64 * len(self.shard_bounds))(*self.shard_bounds)

    @property
    def n_shards(self) -> int:
        return len(self.shard_bounds) - 1

    @property
    def n_phys(self) -> int:
        return int(self.k_pages.shape[0])

    def struct(self) -> _lib.ls_prefix_t:
        s = _lib.ls_prefix_t()
        s.hq, s.hkv, s.d, s.page_size = self.hq, self.hkv, self.d, PAGE
        s.dtype = _dtype_code(self.dtype)
        s.n_shards = self.n_shards
        s.prefix_len = self.prefix_len
        s.n_phys_pages = self.n_phys
        s.page_table = self.page_table.data_ptr() if self.page_table.numel() else None
        s.k_pages = self.k_pages.data_ptr() if self.k_pages.numel() else None
        s.v_pages = self.v_pages.data_ptr() if self.v_pages.numel() else None
        s.shard_page_bounds = C.cast(self._bounds, C.POINTER(C.c_int64))
        s.softmax_scale = float(self.softmax_scale)
        return s


def version() -> int:
    return lib().ls_version()


def capture_pages(k: torch.Tensor, v: torch.Tensor, page_table: torch.Tensor, n_phys: int,
                  page_dtype: torch.dtype | None = None, first_tok: int = 0,
                  k_pages: torch.Tensor | None = None, v_pages: torch.Tensor | None = None,
                  check_table: bool = True):
    """Write prompt keys/values [n_tok, hkv, d] (tokens first_tok ..) into page pools
    [n_phys, hkv, 64, d]; allocates the pools (zeroed) when not given.  check_table first checks
    on the host that the table is one to one into [0, n_phys) (a copy of the table to the host,
    so the stream is synchronised once)."""
    _dev(k, "k")
    _dev(v, "v", dtype=k.dtype, shape=k.shape)
    _dev(page_table, "page_table", dtype=torch.int32)
    n_tok, hkv, d = k.shape
    page_dtype = page_dtype or k.dtype
    if check_table:
        check_page_table(page_table, n_phys)
    if k_pages is None:
        k_pages = torch.zeros((n_phys, hkv, PAGE, d), dtype=page_dtype, device=k.device)
        v_pages = torch.zeros_like(k_pages)
    _dev(k_pages, "k_pages", dtype=page_dtype)
    _dev(v_pages, "v_pages", dtype=page_dtype, shape=k_pages.shape)
    check(lib().ls_capture_pages(_ptr(k), _ptr(v), _dtype_code(k.dtype), n_tok, first_tok, _ptr(page_table),
                                 page_table.numel(), _ptr(k_pages), _ptr(v_pages), _dtype_code(page_dtype),
                                 k_pages.shape[0], hkv, d, PAGE, _stream()))
    return k_pages, v_pages


def gather_pages(pages: torch.Tensor, page_table: torch.Tensor, n_tok: int, first_tok: int = 0):
    """Tokens [first_tok, first_tok + n_tok) of a pool, back in logical order."""
    _dev(pages, "pages")
    _dev(page_table, "page_table", dtype=torch.int32)
    n_phys, hkv, _, d = pages.shape
    out = torch.empty((n_tok, hkv, d), dtype=pages.dtype, device=pages.device)
    check(lib().ls_gather_pages(_ptr(pages), _dtype_code(pages.dtype), _ptr(page_table), page_table.numel(),
                                n_phys, first_tok, n_tok, hkv, d, PAGE, _ptr(out), _stream()))
    return out


def fwd_workspace_bytes(prefix: Prefix, n_rows: int) -> int:
    st = prefix.struct()
    n = lib().ls_fwd_workspace_bytes(C.byref(st), n_rows)
    if n == 0 and n_rows > 0:
        raise LongStrawError(_lib.LS_ERR_INVALID, lib().ls_last_error().decode())
    return n


def bwd_workspace_bytes(prefix: Prefix, n_rows: int) -> int:
    st = prefix.struct()
    n = lib().ls_bwd_workspace_bytes(C.byref(st), n_rows)
    if n == 0 and n_rows > 0:
        raise LongStrawError(_lib.LS_ERR_INVALID, lib().ls_last_error().decode())
    return n


def bwd_ds_workspace_bytes(prefix: Prefix, n_rows: int, key_end: int, heads: int | None = None,
                           parts: int | None = None) -> int:
    """Backward workspace that also holds the block's dS (bf16), so that dQ is formed from it
    rather than recomputed; key_end = q_start + n_rows (the largest over a member's blocks
    sizes one workspace for all of them).  With heads (< hkv) or parts (< n_shards + 1) it is
    sized for chunks of that many kv heads by that many consecutive key parts, which the
    library then runs one after another (ls_bwd_ds_chunk_workspace_bytes)."""
    st = prefix.struct()
    if heads is None and parts is None:
        n = lib().ls_bwd_ds_workspace_bytes(C.byref(st), n_rows, key_end)
    else:
        heads = prefix.hkv if heads is None else heads
        parts = prefix.n_shards + 1 if parts is None else parts
        n = lib().ls_bwd_ds_chunk_workspace_bytes(C.byref(st), n_rows, key_end, heads, parts)
    if n == 0 and n_rows > 0:
        raise LongStrawError(_lib.LS_ERR_INVALID, lib().ls_last_error().decode())
    return n


def check_page_table(page_table: torch.Tensor, n_phys: int) -> None:
    """Raise LongStrawError unless the table maps logical pages one to one into [0, n_phys)
    (ls_check_page_table, on a host copy of the table)."""
    host = page_table.detach().to("cpu", torch.int32).contiguous()
    check(lib().ls_check_page_table(C.c_void_p(host.data_ptr()) if host.numel() else None, host.numel(), n_phys))


def owner_slots(prefix: Prefix, n_rows: int, key_end: int) -> int:
    """Slots of the one-writer counters for a block (ls_debug_owner_slots)."""
    st = prefix.struct()
    n = lib().ls_debug_owner_slots(C.byref(st), n_rows, key_end)
    if n == 0:
        raise LongStrawError(_lib.LS_ERR_INVALID, lib().ls_last_error().decode())
    return n


class OwnerCounts:
    """One-writer counters registered for this thread's backward calls while the context is
    open (ls_debug_set_owner_counts): each call zeroes them, then every writer of a gradient
    half-page or dQ part row adds 1 to its slot.  check() raises if any slot was written
    twice."""

    def __init__(self, n_slots: int, device="cuda"):
        self.counts = torch.zeros((n_slots,), dtype=torch.int32, device=device)

    def __enter__(self):
        check(lib().ls_debug_set_owner_counts(_ptr(self.counts), self.counts.numel()))
        return self

    def __exit__(self, *exc):
        lib().ls_debug_set_owner_counts(None, 0)
        return False

    def check(self, what: str = "backward") -> torch.Tensor:
        """The counters on the host (a synchronisation); raises unless every slot is 0 or 1."""
        c = self.counts.cpu()
        bad = torch.nonzero(c > 1).flatten()
        if bad.numel():
            raise RuntimeError(f"{what}: {bad.numel()} counter slots have more than one writer "
                               f"(first slot {int(bad[0])}, count {int(c[bad[0]])})")
        return c


def ds_fits(nbytes: int, device, fraction: float = 0.9, budget: int | None = None) -> bool:
    """Whether a workspace of nbytes fits in what the device has free (counting the blocks
    torch's allocator holds but does not use), or in `budget` bytes when one is given."""
    if budget is not None:
        return nbytes <= budget
    free, _ = torch.cuda.mem_get_info(device)
    cached = torch.cuda.memory_reserved(device) - torch.cuda.memory_allocated(device)
    return nbytes <= fraction * (free + cached)


def _workspace(nbytes: int, device, given: torch.Tensor | None):
    if given is not None:
        if given.numel() * given.element_size() < nbytes:
            raise LongStrawError(_lib.LS_ERR_WORKSPACE, f"workspace of {nbytes} bytes needed")
        return given
    return torch.empty((max(1, (nbytes + 15) // 16) * 4,), dtype=torch.float32, device=device)


def fwd_parts(prefix: Prefix, n_rows: int, workspace: torch.Tensor):
    """Views of the forward workspace: (o_parts [n_parts, n_rows, hq, d], lse_parts)."""
    n_parts = prefix.n_shards + 1
    n_o = n_parts * n_rows * prefix.hq * prefix.d
    o = workspace[:n_o].view(n_parts, n_rows, prefix.hq, prefix.d)
    lse = workspace[n_o:n_o + n_parts * n_rows * prefix.hq].view(n_parts, n_rows, prefix.hq)
    return o, lse


def replay_fwd(prefix: Prefix, q: torch.Tensor, q_start: int, k_resp: torch.Tensor, v_resp: torch.Tensor,
               workspace: torch.Tensor | None = None, o: torch.Tensor | None = None,
               lse: torch.Tensor | None = None):
    """Forward of response rows [q_start, q_start + n_rows): returns (o, lse, workspace)."""
    _dev(q, "q", dtype=prefix.dtype)
    n_rows = q.shape[0]
    _dev(k_resp, "k_resp", dtype=prefix.dtype)
    _dev(v_resp, "v_resp", dtype=prefix.dtype, shape=k_resp.shape)
    o = torch.empty_like(q) if o is None else _dev(o, "o", dtype=prefix.dtype, shape=q.shape)
    if lse is None:
        lse = torch.empty((n_rows, prefix.hq), dtype=torch.float32, device=q.device)
    _dev(lse, "lse", dtype=torch.float32, shape=(n_rows, prefix.hq))
    ws_bytes = fwd_workspace_bytes(prefix, n_rows)
    ws = _workspace(ws_bytes, q.device, workspace)
    st = prefix.struct()
    check(lib().ls_replay_fwd(C.byref(st), _ptr(q), n_rows, q_start, _ptr(k_resp), _ptr(v_resp), k_resp.shape[0],
                              _ptr(o), _ptr(lse), _ptr(ws), ws.numel() * ws.element_size(), _stream()))
    return o, lse, ws


def score_workspace_bytes(prefix: Prefix, n_members: int, n_rows: int) -> int:
    st = prefix.struct()
    n = lib().ls_score_workspace_bytes(C.byref(st), n_members, n_rows)
    if n == 0 and n_members * n_rows > 0:
        raise LongStrawError(_lib.LS_ERR_INVALID, lib().ls_last_error().decode())
    return n


def score_fwd(prefix: Prefix, q: torch.Tensor, k_resp: torch.Tensor, v_resp: torch.Tensor,
              workspace: torch.Tensor | None = None, o: torch.Tensor | None = None,
              lse: torch.Tensor | None = None):
    """Forward-only scoring of several members' whole responses, batched: q is
    [members, rows, hq, d], k_resp / v_resp [members, rows, hkv, d].  Returns (o, lse, workspace)
    with o [members, rows, hq, d] and lse [members, rows, hq]."""
    _dev(q, "q", dtype=prefix.dtype)
    if q.dim() != 4:
        raise ValueError(f"q must be [members, rows, hq, d], got {tuple(q.shape)}")
    n_members, n_rows = q.shape[0], q.shape[1]
    _dev(k_resp, "k_resp", dtype=prefix.dtype, shape=(n_members, n_rows, prefix.hkv, prefix.d))
    _dev(v_resp, "v_resp", dtype=prefix.dtype, shape=k_resp.shape)
    o = torch.empty_like(q) if o is None else _dev(o, "o", dtype=prefix.dtype, shape=q.shape)
    if lse is None:
        lse = torch.empty((n_members, n_rows, prefix.hq), dtype=torch.float32, device=q.device)
    _dev(lse, "lse", dtype=torch.float32, shape=(n_members, n_rows, prefix.hq))
    ws = _workspace(score_workspace_bytes(prefix, n_members, n_rows), q.device, workspace)
    st = prefix.struct()
    check(lib().ls_score_fwd(C.byref(st), n_members, _ptr(q), n_rows, _ptr(k_resp), _ptr(v_resp), _ptr(o), _ptr(lse),
                             _ptr(ws), ws.numel() * ws.element_size(), _stream()))
    return o, lse, ws


def replay_bwd(prefix: Prefix, q, q_start: int, k_resp, v_resp, o, lse, dout, dk_resp, dv_resp,
               resp_first_touch: bool, dk_pages, dv_pages, shard_first_touch=None,
               workspace: torch.Tensor | None = None, dq: torch.Tensor | None = None, store_ds: bool = False,
               dq_pass: bool = True):
    """Backward of one block: returns dq (float32); accumulates or writes the response and
    prompt key/value gradients in place.  store_ds (when no workspace is given) allocates the
    larger workspace with which the library forms dQ from a stored dS; a given workspace
    selects that path by its size alone.  dq_pass=False runs the key/value gradients only (dQ
    formed by replay_fwd_dq) and returns None."""
    _dev(q, "q", dtype=prefix.dtype)
    n_rows = q.shape[0]
    _dev(o, "o", dtype=prefix.dtype, shape=q.shape)
    _dev(dout, "dout", dtype=prefix.dtype, shape=q.shape)
    _dev(lse, "lse", dtype=torch.float32, shape=(n_rows, prefix.hq))
    _dev(dk_resp, "dk_resp", dtype=torch.float32, shape=k_resp.shape)
    _dev(dv_resp, "dv_resp", dtype=torch.float32, shape=k_resp.shape)
    if prefix.prefix_len > 0:
        _dev(dk_pages, "dk_pages", dtype=torch.float32, shape=prefix.k_pages.shape)
        _dev(dv_pages, "dv_pages", dtype=torch.float32, shape=prefix.k_pages.shape)
    if not dq_pass:
        dq = None
        store_ds = False
    else:
        if dq is None:
            dq = torch.empty(q.shape, dtype=torch.float32, device=q.device)
        _dev(dq, "dq", dtype=torch.float32, shape=q.shape)
    flags = None
    if shard_first_touch is not None:
        flags = (C.c_uint8 * prefix.n_shards)(*[1 if f else 0 for f in shard_first_touch])
    if store_ds and workspace is None:
        ws_bytes = bwd_ds_workspace_bytes(prefix, n_rows, q_start + n_rows)
    else:
        ws_bytes = bwd_workspace_bytes(prefix, n_rows)
    ws = _workspace(ws_bytes, q.device, workspace)
    st = prefix.struct()
    check(lib().ls_replay_bwd(C.byref(st), _ptr(q), n_rows, q_start, _ptr(k_resp), _ptr(v_resp), k_resp.shape[0],
                              _ptr(o), _ptr(lse), _ptr(dout), _ptr(dq) if dq is not None else None,
                              _ptr(dk_resp), _ptr(dv_resp),
                              1 if resp_first_touch else 0, _ptr(dk_pages) if dk_pages is not None else None,
                              _ptr(dv_pages) if dv_pages is not None else None,
                              C.cast(flags, C.c_void_p) if flags is not None else None,
                              _ptr(ws), ws.numel() * ws.element_size(), _stream()))
    return dq


def fwd_dq_workspace_bytes(prefix: Prefix, n_rows: int) -> int:
    st = prefix.struct()
    n = lib().ls_fwd_dq_workspace_bytes(C.byref(st), n_rows)
    if n == 0 and n_rows > 0:
        raise LongStrawError(_lib.LS_ERR_INVALID, lib().ls_last_error().decode())
    return n


def replay_fwd_dq(prefix: Prefix, q: torch.Tensor, q_start: int, k_resp: torch.Tensor, v_resp: torch.Tensor,
                  dout: torch.Tensor, workspace: torch.Tensor | None = None, o: torch.Tensor | None = None,
                  lse: torch.Tensor | None = None, dq: torch.Tensor | None = None):
    """Forward of response rows [q_start, q_start + n_rows) and their dQ for the given dL/dO, in
    one pass over the keys (ls_replay_fwd_dq, bf16): returns (o, lse, dq, workspace).  The key
    and value gradients then come from replay_bwd(..., dq_pass=False)."""
    _dev(q, "q", dtype=prefix.dtype)
    n_rows = q.shape[0]
    _dev(k_resp, "k_resp", dtype=prefix.dtype)
    _dev(v_resp, "v_resp", dtype=prefix.dtype, shape=k_resp.shape)
    _dev(dout, "dout", dtype=prefix.dtype, shape=q.shape)
    o = torch.empty_like(q) if o is None else _dev(o, "o", dtype=prefix.dtype, shape=q.shape)
    if lse is None:
        lse = torch.empty((n_rows, prefix.hq), dtype=torch.float32, device=q.device)
    _dev(lse, "lse", dtype=torch.float32, shape=(n_rows, prefix.hq))
    if dq is None:
        dq = torch.empty(q.shape, dtype=torch.float32, device=q.device)
    _dev(dq, "dq", dtype=torch.float32, shape=q.shape)
    ws = _workspace(fwd_dq_workspace_bytes(prefix, n_rows), q.device, workspace)
    st = prefix.struct()
    check(lib().ls_replay_fwd_dq(C.byref(st), _ptr(q), n_rows, q_start, _ptr(k_resp), _ptr(v_resp), k_resp.shape[0],
                                 _ptr(dout), _ptr(o), _ptr(lse), _ptr(dq), _ptr(ws), ws.numel() * ws.element_size(),
                                 _stream()))
    return o, lse, dq, ws


def lse_merge(o_parts: torch.Tensor, lse_parts: torch.Tensor, out_dtype: torch.dtype = torch.float32,
              bf16_numerator: bool = False):
    """Merge [n_parts, n_rows, d] partial outputs by their LSE [n_parts, n_rows] in float32
    (bf16_numerator: the pages' variant with a BF16 numerator, ls_lse_merge_bf16num)."""
    _dev(o_parts, "o_parts", dtype=torch.float32)
    n_parts, n_rows, d = o_parts.shape
    _dev(lse_parts, "lse_parts", dtype=torch.float32, shape=(n_parts, n_rows))
    o = torch.empty((n_rows, d), dtype=out_dtype, device=o_parts.device)
    lse = torch.empty((n_rows,), dtype=torch.float32, device=o_parts.device)
    fn = lib().ls_lse_merge_bf16num if bf16_numerator else lib().ls_lse_merge
    check(fn(n_parts, n_rows, d, _ptr(o_parts), _ptr(lse_parts), _ptr(o), _dtype_code(out_dtype), _ptr(lse),
             _stream()))
    return o, lse


def profile_begin() -> None:
    """Start timing every library kernel launch with HIP events on its stream."""
    check(lib().ls_profile_begin())


def profile_end() -> dict:
    """Stop timing; returns {kernel name: (launches, total ms)} (waits for the events)."""
    buf = (_lib.ls_kernel_stat_t * 64)()
    n = C.c_int(0)
    check(lib().ls_profile_end(buf, 64, C.byref(n)))
    return {buf[i].name.decode(): (int(buf[i].launches), float(buf[i].total_ms)) for i in range(min(n.value, 64))}
