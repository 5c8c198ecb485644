"""C ABI checks that need no GPU: the library loads, exports every function the header
declares, and rejects bad arguments with the documented code before launching anything."""
import ctypes as C
import os
import re

import pytest

from suffix_attention_amd import _lib
from suffix_attention_amd._lib import (LS_DTYPE_BF16, LS_DTYPE_F32, LS_ERR_INVALID, LS_ERR_UNSUPPORTED,
                                       LS_ERR_WORKSPACE, ls_prefix_t)

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "longstraw.h")

FAKE = 0x10000  # never dereferenced: every call below fails validation first


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ls_[a-z0-9_]+)\s*\(", text)))


def test_header_functions_exported():
    names = declared_functions()
    assert {"ls_capture_pages", "ls_replay_fwd", "ls_replay_bwd", "ls_lse_merge"} <= set(names)
    lib = _lib.lib()
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(_lib._SIG), "binding signatures and header disagree"


def test_version():
    assert _lib.lib().ls_version() == 100


def _prefix(**kw):
    b = (C.c_int64 * 3)(0, 1, 2)
    p = ls_prefix_t()
    p.hq, p.hkv, p.d, p.page_size, p.dtype, p.n_shards = 8, 2, 256, 64, LS_DTYPE_BF16, 2
    p.prefix_len, p.n_phys_pages = 128, 2
    p.page_table = p.k_pages = p.v_pages = FAKE
    p.shard_page_bounds = C.cast(b, C.POINTER(C.c_int64))
    p.softmax_scale = 0.0625
    for k, v in kw.items():
        if k == "bounds":
            b = (C.c_int64 * len(v))(*v)
            p.shard_page_bounds = C.cast(b, C.POINTER(C.c_int64))
        else:
            setattr(p, k, v)
    p._keep = b
    return p


def _fwd(p, n_rows=16, q_start=0, n_resp=16, ws_bytes=1 << 30, ws=FAKE, q=FAKE, o=FAKE, lse=FAKE):
    lib = _lib.lib()
    return lib.ls_replay_fwd(C.byref(p), q, n_rows, q_start, FAKE, FAKE, n_resp, o, lse, ws, ws_bytes, None)


def _err():
    return _lib.lib().ls_last_error().decode()


@pytest.mark.parametrize("kw,code,msg", [
    (dict(hq=7), LS_ERR_INVALID, "multiple of hkv"),
    (dict(d=96), LS_ERR_UNSUPPORTED, "head dim"),
    (dict(page_size=32), LS_ERR_UNSUPPORTED, "page_size"),
    (dict(dtype=5), LS_ERR_UNSUPPORTED, "dtype"),
    (dict(n_shards=0), LS_ERR_INVALID, "n_shards"),
    (dict(n_shards=65), LS_ERR_INVALID, "n_shards"),
    (dict(bounds=[0, 1, 3]), LS_ERR_INVALID, "shard bounds"),
    (dict(n_shards=3, bounds=[0, 2, 1, 2]), LS_ERR_INVALID, "decrease"),
    (dict(page_table=None), LS_ERR_INVALID, "non-NULL"),
    (dict(prefix_len=-1), LS_ERR_INVALID, "prefix_len"),
    (dict(softmax_scale=float("nan")), LS_ERR_INVALID, "softmax_scale"),
    (dict(softmax_scale=-0.5), LS_ERR_INVALID, "softmax_scale"),
])
def test_fwd_rejects_bad_prefix(kw, code, msg):
    assert _fwd(_prefix(**kw)) == code
    assert msg in _err()


def test_fwd_rejects_bad_block():
    p = _prefix()
    assert _fwd(p, n_rows=16, q_start=8, n_resp=20) == LS_ERR_INVALID
    assert "n_resp_keys" in _err()
    assert _fwd(p, n_rows=-1) == LS_ERR_INVALID
    assert _fwd(p, q=None) == LS_ERR_INVALID
    assert _fwd(p, o=None) == LS_ERR_INVALID


def test_workspace_size_and_errors():
    p = _prefix()
    lib = _lib.lib()
    need = lib.ls_fwd_workspace_bytes(C.byref(p), 16)
    assert need == 4 * 3 * 16 * 8 * 257
    assert _fwd(p, ws_bytes=need - 1) == LS_ERR_WORKSPACE
    assert _fwd(p, ws=None) == LS_ERR_WORKSPACE
    nb = lib.ls_bwd_workspace_bytes(C.byref(p), 16)
    # delta, dQ parts, then per kv head and padded group row: (lse2, delta) and bf16 Q, dO rows
    assert nb == 4 * (128 + 3 * 16 * 8 * 256) + (8 + 2 * 2 * 256) * 64 * 2
    assert lib.ls_fwd_workspace_bytes(C.byref(_prefix(hq=7)), 16) == 0
    assert "multiple" in _err()


def test_stored_ds_workspace_size():
    """The backward workspace with room for dS: the recompute workspace rounded up to 256
    bytes, then kv heads x row tiles (group rows padded to 256, 32 per tile) x key slots (128
    per page pair, prompt and response pairs) x 64 bytes; float32 stores none."""
    p = _prefix()
    lib = _lib.lib()
    base = (lib.ls_bwd_workspace_bytes(C.byref(p), 16) + 255) // 256 * 256
    # 16 rows x g 4 = 64 group rows -> 8 row tiles; 2 prompt pages -> 1 pair
    assert lib.ls_bwd_ds_workspace_bytes(C.byref(p), 16, 16) == base + 2 * 8 * 128 * (1 + 1) * 64
    assert lib.ls_bwd_ds_workspace_bytes(C.byref(p), 16, 200) == base + 2 * 8 * 128 * (1 + 2) * 64
    assert lib.ls_bwd_ds_workspace_bytes(C.byref(p), 16, 15) == 0 and "key_end" in _err()
    f = _prefix(dtype=LS_DTYPE_F32)
    assert lib.ls_bwd_ds_workspace_bytes(C.byref(f), 16, 16) == lib.ls_bwd_workspace_bytes(C.byref(f), 16)


def test_score_workspace_and_validation():
    """Batched scoring: the workspace is the forward one for members * rows rows, with shards
    split into page ranges as each member's own replay block would split them; bad sizes,
    missing outputs and short workspaces are rejected before any launch."""
    p = _prefix()
    lib = _lib.lib()
    assert lib.ls_score_workspace_bytes(C.byref(p), 3, 16) == lib.ls_fwd_workspace_bytes(C.byref(p), 48)
    # 1,024 pages in 2 shards: a 16-row block splits them (8 ranges a shard), with or without
    # other members batched beside it
    big = _prefix(prefix_len=65536, n_phys_pages=1024, bounds=[0, 512, 1024])
    parts = 4 * 3 * 16 * 8 * 257
    assert lib.ls_fwd_workspace_bytes(C.byref(big), 16) == parts + 4 * 17 * 16 * 8 * 257
    assert lib.ls_score_workspace_bytes(C.byref(big), 1, 16) == lib.ls_fwd_workspace_bytes(C.byref(big), 16)
    assert lib.ls_score_workspace_bytes(C.byref(big), 3, 16) == 3 * lib.ls_fwd_workspace_bytes(C.byref(big), 16)
    assert lib.ls_score_workspace_bytes(C.byref(p), -1, 16) == 0 and "n_members" in _err()
    need = lib.ls_score_workspace_bytes(C.byref(p), 2, 16)
    score = lambda **kw: lib.ls_score_fwd(C.byref(p), kw.get("m", 2), kw.get("q", FAKE), 16, FAKE, FAKE,  # noqa: E731
                                          kw.get("o", FAKE), FAKE, kw.get("ws", FAKE), kw.get("ws_bytes", need), None)
    assert score(m=-1) == LS_ERR_INVALID
    assert score(q=None) == LS_ERR_INVALID
    assert score(o=None) == LS_ERR_INVALID
    assert score(ws_bytes=need - 1) == LS_ERR_WORKSPACE
    assert score(m=0, ws=None, ws_bytes=0) == 0  # nothing to score


def test_fused_workspace_and_validation():
    """The fused forward + dQ pass: float32 o, A / l and B / l parts of d elements and the LSE
    and delta parts, per part and (row, head); a NULL dout or dq, a short workspace and float32
    pages are rejected before any launch; an empty block does nothing."""
    p = _prefix()
    lib = _lib.lib()
    need = lib.ls_fwd_dq_workspace_bytes(C.byref(p), 16)
    assert need == 4 * 3 * 16 * 8 * (3 * 256 + 2)
    assert lib.ls_fwd_dq_workspace_bytes(C.byref(p), -1) == 0 and "n_rows" in _err()

    def fused(p=p, n_rows=16, dout=FAKE, dq=FAKE, ws_bytes=need):
        return lib.ls_replay_fwd_dq(C.byref(p), FAKE, n_rows, 0, FAKE, FAKE, 16, dout, FAKE, FAKE, dq, FAKE,
                                    ws_bytes, None)
    assert fused(dout=None) == LS_ERR_INVALID and "dout" in _err()
    assert fused(dq=None) == LS_ERR_INVALID
    assert fused(ws_bytes=need - 1) == LS_ERR_WORKSPACE
    f = _prefix(dtype=LS_DTYPE_F32)
    assert fused(p=f, ws_bytes=lib.ls_fwd_dq_workspace_bytes(C.byref(f), 16)) == LS_ERR_UNSUPPORTED
    assert "bf16" in _err()
    assert fused(n_rows=0, ws_bytes=0) == 0


def test_fused_group_refuses_writer_counting():
    """The one-writer counters cover backward calls that form dQ; a fused group forms it in
    the forward, so the driver refuses the combination up front."""
    import types

    from suffix_attention_amd import driver
    with pytest.raises(ValueError):
        driver.GroupReplay(types.SimpleNamespace(n_shards=2), fused=True, check_owners=True)


def test_empty_block_is_a_no_op():
    assert _fwd(_prefix(), n_rows=0, n_resp=0, ws=None, ws_bytes=0) == 0


def test_bwd_rejects_missing_gradients():
    p = _prefix()
    lib = _lib.lib()
    rc = lib.ls_replay_bwd(C.byref(p), FAKE, 16, 0, FAKE, FAKE, 16, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1,
                           None, FAKE, None, FAKE, 1 << 30, None)
    assert rc == LS_ERR_INVALID and "dk_pages" in _err()
    rc = lib.ls_replay_bwd(C.byref(p), FAKE, 16, 0, FAKE, FAKE, 16, FAKE, FAKE, FAKE, FAKE, None, FAKE, 1,
                           FAKE, FAKE, None, FAKE, 1 << 30, None)
    assert rc == LS_ERR_INVALID and "dk_resp" in _err()
    rc = lib.ls_replay_bwd(C.byref(p), FAKE, 16, 0, FAKE, FAKE, 16, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1,
                           FAKE, FAKE, None, FAKE, 100, None)
    assert rc == LS_ERR_WORKSPACE


def test_capture_and_merge_validation():
    lib = _lib.lib()
    # misaligned chunk start
    assert lib.ls_capture_pages(FAKE, FAKE, LS_DTYPE_BF16, 10, 5, FAKE, 4, FAKE, FAKE, LS_DTYPE_BF16, 4, 2, 256,
                                64, None) == LS_ERR_INVALID
    # bf16 -> f32 is not a supported capture
    assert lib.ls_capture_pages(FAKE, FAKE, LS_DTYPE_BF16, 10, 0, FAKE, 4, FAKE, FAKE, LS_DTYPE_F32, 4, 2, 256,
                                64, None) == LS_ERR_UNSUPPORTED
    # tokens past the table
    assert lib.ls_capture_pages(FAKE, FAKE, LS_DTYPE_BF16, 300, 0, FAKE, 4, FAKE, FAKE, LS_DTYPE_BF16, 4, 2, 256,
                                64, None) == LS_ERR_INVALID
    assert lib.ls_capture_pages(FAKE, FAKE, LS_DTYPE_BF16, 0, 0, None, 0, None, None, LS_DTYPE_BF16, 0, 2, 256,
                                64, None) == 0
    assert lib.ls_lse_merge(0, 10, 256, FAKE, FAKE, FAKE, LS_DTYPE_F32, FAKE, None) == LS_ERR_INVALID
    assert lib.ls_lse_merge(2, 10, 6, FAKE, FAKE, FAKE, LS_DTYPE_F32, FAKE, None) == LS_ERR_UNSUPPORTED
    assert lib.ls_lse_merge(2, 10, 256, None, FAKE, FAKE, LS_DTYPE_F32, FAKE, None) == LS_ERR_INVALID
    assert lib.ls_gather_pages(FAKE, 7, FAKE, 4, 4, 0, 10, 2, 256, 64, FAKE, None) == LS_ERR_UNSUPPORTED


def test_profile_begin_end_without_launches():
    from suffix_attention_amd import api
    api.profile_begin()
    assert api.profile_end() == {}
    n = C.c_int(0)
    # end without begin is an error
    assert _lib.lib().ls_profile_end(None, 0, C.byref(n)) == LS_ERR_INVALID


def test_stored_ds_chunk_workspace_sizes():
    """Chunks of h kv heads over all key parts take h heads' share of the dS; one kv head by k key
    parts takes the largest chunk's key slots; invalid chunkings are rejected."""
    p = _prefix()
    lib = _lib.lib()
    base = (lib.ls_bwd_workspace_bytes(C.byref(p), 16) + 255) // 256 * 256
    full = lib.ls_bwd_ds_workspace_bytes(C.byref(p), 16, 16)
    assert lib.ls_bwd_ds_chunk_workspace_bytes(C.byref(p), 16, 16, 2, 3) == full
    assert lib.ls_bwd_ds_chunk_workspace_bytes(C.byref(p), 16, 16, 1, 3) == base + 8 * 128 * 2 * 64
    # shards of one page each and the response (one pair): every single part is one page pair
    assert lib.ls_bwd_ds_chunk_workspace_bytes(C.byref(p), 16, 16, 1, 1) == base + 8 * 128 * 1 * 64
    assert lib.ls_bwd_ds_chunk_workspace_bytes(C.byref(p), 16, 16, 2, 1) == 0 and "all parts" in _err()
    assert lib.ls_bwd_ds_chunk_workspace_bytes(C.byref(p), 16, 16, 3, 3) == 0
    assert lib.ls_bwd_ds_chunk_workspace_bytes(C.byref(p), 16, 16, 1, 0) == 0


def test_check_page_table():
    lib = _lib.lib()

    def chk(entries, n_phys):
        arr = (C.c_int32 * max(1, len(entries)))(*entries)
        return lib.ls_check_page_table(C.cast(arr, C.c_void_p), len(entries), n_phys)

    assert chk([3, 0, 2, 1], 4) == 0
    assert chk([3, 0, 2], 6) == 0
    assert chk([0, 1, 1, 2], 4) == LS_ERR_INVALID and "page_table[2]" in _err()
    assert chk([0, 4], 4) == LS_ERR_INVALID and "outside" in _err()
    assert chk([0, -2], 4) == LS_ERR_INVALID
    assert chk([0, 1, 2], 2) == LS_ERR_INVALID
    assert lib.ls_check_page_table(None, 0, 0) == 0
    assert lib.ls_check_page_table(None, 3, 3) == LS_ERR_INVALID


def test_binding_checks_tables_before_capture():
    """api.capture_pages checks the table on the host before anything is launched."""
    import torch

    from suffix_attention_amd import api
    with pytest.raises(_lib.LongStrawError, match="already mapped"):
        api.check_page_table(torch.tensor([0, 2, 2], dtype=torch.int32), 3)
    api.check_page_table(torch.tensor([2, 0, 1], dtype=torch.int32), 3)



def test_owner_counter_slots_and_registration():
    """The one-writer counter layout documented in the header: prompt half-pages, response
    half-pages, dQ part rows; registration rejects a buffer of zero slots; a registered
    backward checks the size (and the dtype) before anything is launched."""
    lib = _lib.lib()
    p = _prefix()  # hq 8, hkv 2, 2 shards, 2 physical pages
    n_rows, key_end = 16, 80
    want = 2 * 2 * 2 + ((key_end + 63) // 64) * 2 * 2 + 3 * n_rows * 8
    assert lib.ls_debug_owner_slots(C.byref(p), n_rows, key_end) == want
    assert lib.ls_debug_owner_slots(C.byref(_prefix(hkv=3)), n_rows, key_end) == 0 and "hq" in _err()
    assert lib.ls_debug_owner_slots(C.byref(p), 20, 10) == 0
    assert lib.ls_debug_set_owner_counts(FAKE, 0) == LS_ERR_INVALID
    try:
        assert lib.ls_debug_set_owner_counts(FAKE, 10) == 0
        rc = lib.ls_replay_bwd(C.byref(p), FAKE, 16, 0, FAKE, FAKE, 16, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1,
                               FAKE, FAKE, None, FAKE, 1 << 30, None)
        assert rc == LS_ERR_INVALID and "slots needed" in _err()
        rc = lib.ls_replay_bwd(C.byref(_prefix(dtype=LS_DTYPE_F32)), FAKE, 16, 0, FAKE, FAKE, 16, FAKE, FAKE, FAKE,
                               FAKE, FAKE, FAKE, 1, FAKE, FAKE, None, FAKE, 1 << 30, None)
        assert rc == LS_ERR_UNSUPPORTED and "bf16" in _err()
    finally:
        assert lib.ls_debug_set_owner_counts(None, 0) == 0


def test_owner_counts_check_flags_a_second_writer():
    """OwnerCounts.check passes counters of 0 and 1 and names the first slot written twice."""
    import torch

    from suffix_attention_amd import api
    oc = api.OwnerCounts(12, device="cpu")
    oc.counts[[0, 3, 4]] = 1
    assert int(oc.check().sum()) == 3
    oc.counts[7] = 2
    with pytest.raises(RuntimeError, match="first slot 7, count 2"):
        oc.check()
    assert torch.equal(oc.counts[:7], torch.tensor([1, 0, 0, 1, 1, 0, 0], dtype=torch.int32))


def test_trace_ranges_nest_and_pop_on_errors():
    """roctx ranges (a no-op where the roctx library cannot be loaded) nest, and a range is
    popped when its body raises."""
    from suffix_attention_amd import trace
    with trace.trace_range("outer"):
        with trace.trace_range("inner"):
            pass
    with pytest.raises(ValueError):
        with trace.trace_range("raises"):
            raise ValueError("x")
    if trace.available():
        # the library's own depth counter: pushing returns the depth before the push
        lib = trace._roctx()
        depth = lib.roctxRangePushA(b"probe")
        lib.roctxRangePop()
        assert depth == 0, depth
