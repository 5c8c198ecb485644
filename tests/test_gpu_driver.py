"""The serial group driver against the oracle, end to end.

G members are replayed one after another over one captured prompt, each in reverse blocks
(the last, ragged block first), with the prompt split into uneven shards behind a permuted page
table (LongStraw digest, "Method", step 3: replay one member, backpropagate, accumulate, free,
then the next; explainer, "Two incompatible architectures, same transaction": response blocks
replayed in reverse, K/V gradient pages allocated when a backward first touches them).  Every
member's O, LSE, dQ and response-key gradients are compared with the oracle over that member's
whole response, and the prompt gradient pages the group accumulated (in logical order) with the
oracle's prompt gradients summed over the members.  Nothing here compares the driver with
itself.
"""
import numpy as np
import pytest
import torch

from _cases import assert_close, log, np32
from oracle import attention as orc
from suffix_attention_amd import api, datagen, driver

pytestmark = pytest.mark.gpu

# 2,000 prompt tokens (31 full pages and a partial one) in 3 uneven shards with odd page bounds,
# a pool with 3 pages more than the prompt uses, behind a seeded permutation; 3 members with
# 300-token responses in reverse blocks of 128 rows (rows 256..299 first, 44 rows).
P, R, B, HQ, HKV, D, G = 2000, 300, 128, 24, 4, 256, 3
BOUNDS = [0, 5, 19, 32]
N_PAGES, N_PHYS = 32, 35


def _inputs():
    s = lambda tag: 104729 + tag  # noqa: E731
    table = datagen.page_table(N_PHYS, s(1))[:N_PAGES].to(torch.int32)
    kp = datagen.normal((P, HKV, D), s(2), torch.bfloat16)
    vp = datagen.normal((P, HKV, D), s(3), torch.bfloat16)
    members = []
    for i in range(G):
        members.append(dict(q=datagen.normal((R, HQ, D), s(10 + 4 * i), torch.bfloat16),
                            kr=datagen.normal((R, HKV, D), s(11 + 4 * i), torch.bfloat16),
                            vr=datagen.normal((R, HKV, D), s(12 + 4 * i), torch.bfloat16),
                            do=datagen.normal((R, HQ, D), s(13 + 4 * i), torch.bfloat16)))
    return table, kp, vp, members


def _oracle(kp, vp, members):
    """Per member: the oracle over the whole response (q_start = 0, delta from the oracle's own
    output rounded to bf16, as the library stores it); and the prompt gradients summed over the
    members."""
    f = lambda t: t.float().numpy()  # noqa: E731
    refs, dkp, dvp = [], 0.0, 0.0
    for m in members:
        O, L = orc.forward(f(m["q"]), f(kp), f(vp), f(m["kr"]), f(m["vr"]), 0)
        g = orc.backward(f(m["q"]), f(kp), f(vp), f(m["kr"]), f(m["vr"]), f(m["do"]), 0,
                         o=orc.round_bf16(O), lse=L)
        refs.append(dict(o=O, lse=L, dq=g["dq"], dkr=g["dkr"], dvr=g["dvr"]))
        dkp = dkp + g["dkp"]
        dvp = dvp + g["dvp"]
    return refs, dkp, dvp


def _logical(pages: torch.Tensor, table: torch.Tensor) -> np.ndarray:
    pg = np32(pages)
    t = np.arange(P)
    return pg[table.numpy()[t // 64], :, t % 64, :]


def _poison_allocator():
    """Leave NaN-filled blocks in torch's caching allocator, so that the driver's torch.empty
    buffers (gradient pages, outputs, workspaces) start as NaN: a first touch that misses an
    element, or a workspace slot read before it is written, shows up as a non-finite result."""
    junk = [torch.full((n,), float("nan"), dtype=torch.float32, device="cuda")
            for n in (1 << 26, 1 << 24, 1 << 22, 1 << 20, 1 << 18)]
    del junk


def _check_group(grp, results, refs, dkp_ref, dvp_ref, table):
    for i, (r, ref) in enumerate(zip(results, refs)):
        log(f"  member {i}")
        assert_close("O", np32(r.o), ref["o"])
        assert_close("LSE", np32(r.lse), ref["lse"])
        assert_close("dQ", np32(r.dq), ref["dq"])
        assert_close("dK_resp", np32(r.dk_resp), ref["dkr"])
        assert_close("dV_resp", np32(r.dv_resp), ref["dvr"])
    log("  prompt gradient pages summed over the members")
    assert_close("dK_prompt", _logical(grp.dk_pages, table), dkp_ref)
    assert_close("dV_prompt", _logical(grp.dv_pages, table), dvp_ref)


@pytest.fixture(scope="module")
def group_case():
    table, kp, vp, members = _inputs()
    refs, dkp, dvp = _oracle(kp, vp, members)
    dev = "cuda"
    k_pages, v_pages = api.capture_pages(kp.to(dev), vp.to(dev), table.to(dev), N_PHYS)
    pre = api.Prefix(HQ, HKV, D, torch.bfloat16, P, table.to(dev), k_pages, v_pages, list(BOUNDS))
    gpu_members = [{k: v.to(dev) for k, v in m.items()} for m in members]
    return dict(table=table, pre=pre, members=gpu_members, host_members=members, kp=kp, vp=vp, refs=refs,
                dkp=dkp, dvp=dvp)


def _budget(pre, heads, parts):
    """Device-memory budget that holds the workspace of exactly this chunking for every block."""
    blocks = [(b * B, min(R, (b + 1) * B)) for b in range((R + B - 1) // B)]
    return max(api.bwd_ds_workspace_bytes(pre, e - a, e, heads=heads, parts=parts) for a, e in blocks)


@pytest.mark.parametrize("form", ["stored dS, 1 kv head", "stored dS, 1 kv head x 2 key parts",
                                  "stored dS, all", "recompute",
                                  "stored dS, 1 kv head x 2 key parts, writers counted",
                                  "fused forward + dQ"])
def test_group_replay_matches_oracle(group_case, form):
    """The writers-counted form runs every backward with the one-writer counters registered
    (the driver raises if any gradient half-page or dQ part row gets two writers) and must
    still match the oracle.  The fused form forms dQ in the forward (ls_replay_fwd_dq) from the
    unrounded O; against the oracle's dQ from the bf16-rounded O it stays within the same
    bounds."""
    c = group_case
    pre = c["pre"]
    kw, plan = {
        "stored dS, 1 kv head": (dict(ds_budget=_budget(pre, 1, 4)), driver.BwdPlan(1, 4)),
        "stored dS, 1 kv head x 2 key parts": (dict(ds_budget=_budget(pre, 1, 2)), driver.BwdPlan(1, 2)),
        "stored dS, all": (dict(store_ds=True), driver.BwdPlan(HKV, 4)),
        "recompute": (dict(store_ds=False), driver.BwdPlan(0, 0)),
        "stored dS, 1 kv head x 2 key parts, writers counted": (
            dict(ds_budget=_budget(pre, 1, 2), check_owners=True), driver.BwdPlan(1, 2)),
        "fused forward + dQ": (dict(fused=True), driver.BwdPlan(0, 0)),
    }[form]
    log(f"case: group of {G} members P={P} S=3 {BOUNDS} R={R} B={B} ({form})")
    _poison_allocator()
    grp, results = driver.replay_group(pre, c["members"], B, **kw)
    torch.cuda.synchronize()
    assert grp.plan == plan, grp.plan
    assert all(r.plan == plan for r in results)
    _check_group(grp, results, c["refs"], c["dkp"], c["dvp"], c["table"])


def test_prefix_reuse_cycles_match_oracle(group_case):
    """Consecutive optimizer cycles over one capture: each cycle is a fresh group whose gradient
    pages are allocated at its first backward; every cycle matches the oracle's summed gradients
    (and the previous cycle, bit for bit)."""
    c = group_case
    pre = c["pre"]
    log(f"case: 3 reuse cycles of G={G} over one capture, stored dS in 1-kv-head chunks")
    prev = None
    for cycle in range(3):
        _poison_allocator()
        grp, results = driver.replay_group(pre, c["members"], B, ds_budget=_budget(pre, 1, 4))
        torch.cuda.synchronize()
        log(f"  cycle {cycle}")
        _check_group(grp, results, c["refs"], c["dkp"], c["dvp"], c["table"])
        # the pages the table maps (the pool's unmapped pages hold no gradient and are never written)
        mapped = pre.page_table.long()
        if prev is not None:
            assert torch.equal(grp.dk_pages[mapped], prev[0]) and torch.equal(grp.dv_pages[mapped], prev[1])
        prev = (grp.dk_pages[mapped].clone(), grp.dv_pages[mapped].clone())
        del grp, results


def test_gradient_pages_are_allocated_at_the_first_backward(group_case):
    """Lazy gradient pages: none exist before the group's first backward, and they are written
    (not added to) by it, whatever the memory held before; blocks run last first."""
    c = group_case
    pre = c["pre"]
    m = c["members"][0]
    grp = driver.GroupReplay(pre, store_ds=True)
    seen = []

    def on_block(rows):
        seen.append((rows, grp.dk_pages is not None))

    assert grp.dk_pages is None and grp.plan is None
    _poison_allocator()
    r = grp.replay_member(m["q"], m["kr"], m["vr"], m["do"], B, on_block=on_block)
    torch.cuda.synchronize()
    assert [s_[0] for s_ in seen] == [(256, 300), (128, 256), (0, 128)], seen   # reverse order, ragged first
    assert all(s_[1] for s_ in seen)
    ref = c["refs"][0]
    f = lambda t: t.float().numpy()  # noqa: E731
    h = c["host_members"][0]
    g = orc.backward(f(h["q"]), f(c["kp"]), f(c["vp"]), f(h["kr"]), f(h["vr"]), f(h["do"]), 0,
                     o=orc.round_bf16(ref["o"]), lse=ref["lse"])
    assert_close("dK_prompt", _logical(grp.dk_pages, c["table"]), g["dkp"])
    assert_close("dV_prompt", _logical(grp.dv_pages, c["table"]), g["dvp"])
    assert_close("dQ", np32(r.dq), ref["dq"])
