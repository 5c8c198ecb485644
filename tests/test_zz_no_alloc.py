"""The no-allocation forward (ls_replay_fwd_noalloc, for callers that cannot allocate device memory)
against the allocating forward (ls_replay_fwd) through the C ABI: the same kernels, so O and LSE
must be equal bit for bit, on two calls in a row whose second is smaller (the scratch array
keeps the first call's contents), for bf16 and float32, and for small blocks over a long prompt
(whose shards split into page ranges); and a block whose forward workspace is larger than the
scratch array is refused before any launch."""
import ctypes as C

import pytest
import torch

from _cases import Case, log
from suffix_attention_amd import _lib, api

pytestmark = pytest.mark.gpu

SCRATCH = 256 << 20  # LS_NOALLOC_SCRATCH_BYTES


def _noalloc(pre, q, q_start, kr, vr):
    o = torch.empty_like(q)
    lse = torch.empty((q.shape[0], pre.hq), dtype=torch.float32, device=q.device)
    st = pre.struct()
    rc = _lib.lib().ls_replay_fwd_noalloc(C.byref(st), C.c_void_p(q.data_ptr()), q.shape[0], q_start,
                                          C.c_void_p(kr.data_ptr()), C.c_void_p(vr.data_ptr()), kr.shape[0],
                                          C.c_void_p(o.data_ptr()), C.c_void_p(lse.data_ptr()),
                                          C.c_void_p(torch.cuda.current_stream().cuda_stream))
    return rc, o, lse


@pytest.mark.parametrize("dtype,shape", [(torch.bfloat16, (3000, 512, 24, 4, 256, 3)),
                                         (torch.float32, (700, 96, 4, 1, 64, 2)),
                                         # small blocks over a long prompt: the shards split into
                                         # page ranges, whose results also live in the scratch array
                                         (torch.bfloat16, (65536, 64, 6, 2, 256, 2))])
def test_noalloc_forward_equals_the_allocating_forward(dtype, shape):
    P, R, hq, hkv, d, S = shape
    c = Case(P, R, hq, hkv, d, dtype, seed=41, S=S)
    pre = c.prefix()
    kr, vr = c.kr.to("cuda"), c.vr.to("cuda")
    for q0, n in ((R // 8, R - R // 8), (10, 37)):
        log(f"case: no-allocation forward {dtype} P={P} S={S} hq={hq} hkv={hkv} d={d} rows [{q0}, {q0 + n})")
        assert api.fwd_workspace_bytes(pre, n) <= SCRATCH
        q = c.q[q0:q0 + n].to("cuda").contiguous()
        o_ref, lse_ref, _ = api.replay_fwd(pre, q, q0, kr, vr)
        rc, o, lse = _noalloc(pre, q, q0, kr, vr)
        torch.cuda.synchronize()
        assert rc == 0, _lib.lib().ls_last_error().decode()
        assert torch.equal(o, o_ref) and torch.equal(lse, lse_ref)


def test_noalloc_refuses_blocks_larger_than_its_scratch():
    c = Case(640, 1300, 24, 4, 256, torch.bfloat16, seed=43, S=8)
    pre = c.prefix()
    n = 1300  # 9 parts x 24 heads x 257 floats x 4 bytes = 222 kB per row: 289 MB > 256 MiB (1,208 rows)
    assert api.fwd_workspace_bytes(pre, n) > SCRATCH
    q = c.q.to("cuda")
    rc, _, _ = _noalloc(pre, q, 0, c.kr.to("cuda"), c.vr.to("cuda"))
    assert rc == _lib.LS_ERR_WORKSPACE
    assert "split the block" in _lib.lib().ls_last_error().decode()
