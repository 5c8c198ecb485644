"""The fused forward + dQ pass (ls_replay_fwd_dq) and the key/value-only backward that follows it
(ls_replay_bwd with dq = NULL), through the C ABI, against the oracle element by element.

The fused pass defines dQ with delta = sum_j P_ij dP_ij = dO_i . O_i on the exact output (it
never rounds O before using it), so its reference is the oracle's backward with the oracle's
exact O; O and LSE are the oracle's forward."""
import numpy as np
import pytest
import torch

from _cases import Case, assert_close, log, np32
from suffix_attention_amd import api

pytestmark = pytest.mark.gpu


def run_fused(c: Case, q_start: int, n_rows: int, prefix=None):
    """The fused pass, then the backward without dQ; returns the results and the fused
    workspace's per-part O and LSE."""
    pre = prefix or c.prefix()
    dev = "cuda"
    q = c.q[q_start:q_start + n_rows].to(dev).contiguous()
    do = c.do[q_start:q_start + n_rows].to(dev).contiguous()
    kr, vr = c.kr.to(dev), c.vr.to(dev)
    o, lse, dq, ws = api.replay_fwd_dq(pre, q, q_start, kr, vr, do)
    n_parts = pre.n_shards + 1
    rows = n_rows * c.hq
    pe = n_parts * rows * c.d
    o_parts = ws[:pe].view(n_parts, n_rows, c.hq, c.d).clone()
    lse_parts = ws[3 * pe:3 * pe + n_parts * rows].view(n_parts, n_rows, c.hq).clone()
    dk_r = torch.full(kr.shape, float("nan"), dtype=torch.float32, device=dev)
    dv_r = torch.full(kr.shape, float("nan"), dtype=torch.float32, device=dev)
    dk_p = torch.full(pre.k_pages.shape, float("nan"), dtype=torch.float32, device=dev)
    dv_p = torch.full(pre.k_pages.shape, float("nan"), dtype=torch.float32, device=dev)
    r = api.replay_bwd(pre, q, q_start, kr, vr, o, lse, do, dk_r, dv_r, True, dk_p, dv_p,
                       shard_first_touch=[True] * pre.n_shards, dq_pass=False)
    assert r is None
    torch.cuda.synchronize()
    return dict(o=o, lse=lse, dq=dq, dkr=dk_r, dvr=dv_r, dk_pages=dk_p, dv_pages=dv_p, o_parts=o_parts,
                lse_parts=lse_parts, prefix=pre)


def check_fused(c: Case, q_start: int, n_rows: int, res=None, parts=True, dq_atol=2e-2):
    """dq_atol: the max-abs bound of dQ (inputs scaled away from N(0, 1) scale dQ with them)."""
    res = res or run_fused(c, q_start, n_rows)
    ref = c.oracle(q_start, n_rows)  # exact O used for delta
    assert_close("O", np32(res["o"]), ref["o"])
    assert_close("LSE", np32(res["lse"]), ref["lse"])
    assert_close("dQ", np32(res["dq"]), ref["dq"], atol=dq_atol)
    # the key and value gradients take delta from the stored (bf16) O, as the backward does
    ref_b = c.oracle(q_start, n_rows, o_used=c.stored(ref["o"]))
    kend = q_start + n_rows
    assert_close("dK_resp", np32(res["dkr"])[:kend], ref_b["dkr"][:kend])
    assert_close("dV_resp", np32(res["dvr"])[:kend], ref_b["dvr"][:kend])
    assert np.all(np32(res["dkr"])[kend:] == 0) and np.all(np32(res["dvr"])[kend:] == 0)
    if c.P > 0:
        assert_close("dK_prompt", c.logical(res["dk_pages"]), ref_b["dkp"])
        assert_close("dV_prompt", c.logical(res["dv_pages"]), ref_b["dvp"])
    if parts:
        Op, Lp = c.oracle_parts(q_start, n_rows)
        gop, glp = np32(res["o_parts"]), np32(res["lse_parts"])
        for p in range(Op.shape[0]):
            empty = np.isneginf(Lp[p])
            assert np.array_equal(np.isneginf(glp[p]), empty), f"part {p}: empty rows differ"
            if np.all(empty):
                assert np.all(gop[p] == 0)
                continue
            assert_close(f"O_part{p}", gop[p], Op[p])
            assert_close(f"LSE_part{p}", glp[p][~empty], Lp[p][~empty])
    return res


@pytest.mark.parametrize("d", [64, 128, 256])
def test_fused_all_head_dims(d):
    log(f"case: fused bf16 P=700 R=160 hq=6 hkv=2 d={d} S=3 rows [32, 128)")
    check_fused(Case(700, 160, 6, 2, d, torch.bfloat16, seed=2, S=3), 32, 96)


def test_fused_gqa6_ragged_blocks():
    """24/4/256 with a ragged prompt tail; 1,200 group rows, the last 64-row tile three-quarters full."""
    log("case: fused bf16 P=1000 R=300 hq=24 hkv=4 d=256 S=8 rows [100, 300)")
    check_fused(Case(1000, 300, 24, 4, 256, torch.bfloat16, seed=3, S=8), 100, 200)


def test_fused_uneven_and_empty_shards():
    log("case: fused bf16 P=1280 bounds [0,0,3,3,11,20] rows [0, 64)")
    check_fused(Case(1280, 64, 12, 4, 256, torch.bfloat16, seed=4, bounds=[0, 0, 3, 3, 11, 20]), 0, 64)


def test_fused_promptless_and_single_row():
    log("case: fused bf16 P=0 R=200 rows [72, 200)")
    check_fused(Case(0, 200, 6, 2, 256, torch.bfloat16, seed=6, S=1), 72, 128)
    log("case: fused bf16 P=333 R=50 rows [49, 50)")
    check_fused(Case(333, 50, 6, 2, 128, torch.bfloat16, seed=7, S=2), 49, 1)


def test_fused_rescales_as_the_maximum_grows():
    """Prompt keys scaled up page after page, so every row's maximum keeps growing and the pass
    moves its reference (and rescales its three accumulators) many times.  dQ = scale sum dS K
    grows with the keys: its largest element is 6.5 here against 0.45 in the unscaled d = 128
    case, so its max-abs bound is ten times the default; the relative bound is the default."""
    c = Case(64 * 24, 96, 6, 2, 128, torch.bfloat16, seed=8, S=2)
    ramp = torch.linspace(0.5, 3.0, c.P).view(-1, 1, 1)
    c.kp = (c.kp.float() * ramp).to(torch.bfloat16)
    log("case: fused bf16 P=1536 (keys ramped x0.5..x3) R=96 hq=6 hkv=2 d=128 rows [0, 96)")
    check_fused(c, 0, 96, dq_atol=10 * 2e-2)


def test_fused_agrees_with_the_two_pass_path():
    """O, LSE and dQ as ls_replay_fwd + ls_replay_bwd give them, to the rounding both carry; and
    given the same O and LSE, the backward without dQ forms bit for bit the key and value
    gradients of the recomputing backward."""
    c = Case(1000, 200, 24, 4, 256, torch.bfloat16, seed=9, S=3)
    log("case: fused vs two-pass, bf16 P=1000 R=200 hq=24 hkv=4 d=256 rows [40, 200)")
    pre = c.prefix()
    f = run_fused(c, 40, 160, prefix=pre)
    t = c.gpu(40, 160, prefix=pre)
    # each path is within the suite's bounds of the oracle (the tests above and
    # test_gpu_parity.py); between them the same bounds apply
    assert_close("O", np32(f["o"]), np32(t["o"]).astype(np.float64))
    assert_close("LSE", np32(f["lse"]), np32(t["lse"]).astype(np.float64))
    assert_close("dQ", np32(f["dq"]), np32(t["dq"]).astype(np.float64))
    dev = "cuda"
    q = c.q[40:200].to(dev).contiguous()
    do = c.do[40:200].to(dev).contiguous()
    kr, vr = c.kr.to(dev), c.vr.to(dev)
    g = {k: torch.zeros_like(f[k]) for k in ("dkr", "dvr", "dk_pages", "dv_pages")}
    api.replay_bwd(pre, q, 40, kr, vr, f["o"], f["lse"], do, g["dkr"], g["dvr"], True, g["dk_pages"],
                   g["dv_pages"], shard_first_touch=[True] * pre.n_shards)
    torch.cuda.synchronize()
    for k in g:
        assert torch.equal(f[k], g[k]), k


def test_fused_is_deterministic():
    c = Case(900, 120, 24, 4, 256, torch.bfloat16, seed=10, S=4)
    log("case: fused determinism, bf16 P=900 R=120 rows [0, 120)")
    pre = c.prefix()
    a = run_fused(c, 0, 120, prefix=pre)
    b = run_fused(c, 0, 120, prefix=pre)
    for k in ("o", "lse", "dq", "dkr", "dvr", "dk_pages", "dv_pages"):
        assert torch.equal(a[k], b[k]), k


def test_fused_rejects_float32_pages():
    c = Case(200, 40, 4, 2, 64, torch.float32, seed=12, S=1)
    pre = c.prefix()
    q = c.q[:40].cuda()
    with pytest.raises(api.LongStrawError):
        api.replay_fwd_dq(pre, q, 0, c.kr.cuda(), c.vr.cuda(), c.do[:40].cuda())
